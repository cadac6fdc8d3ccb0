// Log-sum-exp merge of the raw bf16 partials left by the tuned decode kernel (the
// key range of a sequence split over several work-groups): for each query
// row, M = max_k m_k, L = sum_k 2^(m_k - M) l_k, o = sum_k 2^(m_k - M) O_k / L,
// lse = (M + log2 L) ln 2.  A piece that saw no key (l_k = 0) has weight 0.
//
// One work-group per (sequence, 4 rows), one wave per row: lane i owns latent
// dims 4i .. 4i+3 and 256 + 4i .. +3, so each load instruction reads 1 KB of
// one row contiguously, and the loads of four pieces are in flight at once.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kDc = 512;
constexpr int kGroup = 4;   // pieces whose loads are in flight together

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__global__ void __launch_bounds__(256) combine_stream_kernel(const uint16_t* __restrict__ ws_o,
                                                             const float* __restrict__ ws_stats,
                                                             const int32_t* __restrict__ seqlens, int n_seq,
                                                             int rows_per_seq, SplitLayout lay,
                                                             uint16_t* __restrict__ o_lat, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const int r = blockIdx.y * kRowsPerBlock + wave;
  if (r >= rows_per_seq) return;
  // Each wave finds its sequence's pieces by itself (no barrier): tiles before
  // sequence b and in total, with the decode kernel's clamped lengths.
  int before = 0, all = 0;
  for (int i = lane; i < n_seq; i += 64) {
    const int32_t L = min(max(seqlens[i], 0), lay.max_len);
    const int nt = (L + lay.tile - 1) / lay.tile;
    all += nt;
    if (i < b) before += nt;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    before += __shfl_xor(before, off, 64);
    all += __shfl_xor(all, off, 64);
  }
  const int64_t total = all;
  const int32_t Lb = min(max(seqlens[b], 0), lay.max_len);
  const int64_t nb = (Lb + lay.tile - 1) / lay.tile;
  if (nb == 0) return;
  const int64_t wf = unit_of_tile(before, total, lay.n_splits);
  const int64_t wl = unit_of_tile(before + nb - 1, total, lay.n_splits);
  if (wf == wl) return;                        // the decode kernel wrote this sequence
  const int64_t count = wl - wf + 1;

  // Online merge over the pieces, four at a time: the stats and values of the
  // group are loaded before any is used (one memory latency per group), then
  // folded in against a running maximum m:
  //   acc <- acc 2^(m - m') + 2^(m_k - m') O_k,  tot likewise with l_k.
  // Pieces are taken 64 at a time, lane j telling whether unit wf + k0 + j
  // owns a tile (a unit that owns none left nothing in its slot).
  float m = -INFINITY, tot = 0.f;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int64_t k64 = 0; k64 < count; k64 += 64) {
    const int64_t w_l = wf + k64 + lane;
    const bool owns = k64 + lane < count &&
                      unit_first_tile(w_l, total, lay.n_splits) < unit_first_tile(w_l + 1, total, lay.n_splits);
    const uint64_t owners = __ballot(owns);
    const int64_t n_here = min(count - k64, (int64_t)64);
    for (int k0 = 0; k0 < n_here; k0 += kGroup) {
      f32x2 st[kGroup];
      u32x2 raw[kGroup][2];   // 4 bf16 each
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        if (k0 + j < n_here) {
          const int64_t row = (wf + k64 + k0 + j + b) * rows_per_seq + r;
          st[j] = *(const f32x2*)(ws_stats + row * 2);
          const u32x2* src = (const u32x2*)(ws_o + row * kDc) + lane;
          raw[j][0] = src[0];
          raw[j][1] = src[64];
        }
      }
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        if (k0 + j >= n_here) break;
        if (!((owners >> (k0 + j)) & 1) || !(st[j][1] > 0.f)) continue;
        const float mn = fmaxf(m, st[j][0]);
        const float keep = exp2f(m - mn);          // 0 while nothing is accumulated (m = -inf)
        const float wgt = exp2f(st[j][0] - mn);
        tot = fmaf(tot, keep, wgt * st[j][1]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w2 = raw[j][h][e >> 1];
            const float x = __uint_as_float((e & 1) ? (w2 & 0xffff0000u) : (w2 << 16));
            acc[h][e] = fmaf(acc[h][e], keep, wgt * x);
          }
        m = mn;
      }
    }
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  u32x2* dst = (u32x2*)(o_lat + ((int64_t)b * rows_per_seq + r) * kDc) + lane;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x2 o;
    o[0] = (uint32_t)f32_to_bf16_bits(acc[h][0] * inv) | ((uint32_t)f32_to_bf16_bits(acc[h][1] * inv) << 16);
    o[1] = (uint32_t)f32_to_bf16_bits(acc[h][2] * inv) | ((uint32_t)f32_to_bf16_bits(acc[h][3] * inv) << 16);
    dst[64 * h] = o;
  }
  if (lane == 0)
    lse[(int64_t)b * rows_per_seq + r] = tot > 0.f ? (m + log2f(tot)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

mla_status launch_combine_stream(const mla_dims& d, const DecodePlan& plan, int32_t n_seq, int32_t q_per_seq,
                                 const int32_t* seqlens, const void* ws, void* o_lat, float* lse, hipStream_t st) {
  const int rows = q_per_seq * d.n_heads;
  const uint16_t* ws_o = static_cast<const uint16_t*>(ws);
  const float* ws_stats = static_cast<const float*>(ws) + plan.ws_stats_offset_floats;
  dim3 grid(n_seq, (rows + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(combine_stream_kernel, grid, dim3(256), 0, st, ws_o, ws_stats, seqlens, n_seq, rows,
                     plan.layout, static_cast<uint16_t*>(o_lat), lse);
  return launch_status();
}

}  // namespace mla
