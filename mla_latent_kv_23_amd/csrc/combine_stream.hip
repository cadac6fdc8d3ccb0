// Log-sum-exp merge of the raw partials left by the tuned decode kernel (the
// key range of a sequence split over several work-groups): for each query
// row, M = max_k m_k, L = sum_k 2^(m_k - M) l_k, o = sum_k 2^(m_k - M) O_k / L,
// lse = (M + log2 L) ln 2.  A piece that saw no key (l_k = 0) has weight 0.
//
// One work-group per (sequence, 16 rows); thread t owns row t/16 and 32
// consecutive latent dims, so each row's 2 KB per partial is read by 16
// consecutive lanes.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kRowsPerBlock = 16;
constexpr int kDc = 512;
constexpr int kGroup = 4;   // pieces whose loads are in flight together

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) combine_stream_kernel(const float* __restrict__ ws_o,
                                                             const float* __restrict__ ws_stats,
                                                             const int32_t* __restrict__ seqlens, int n_seq,
                                                             int rows_per_seq, SplitLayout lay,
                                                             uint16_t* __restrict__ o_lat, float* __restrict__ lse) {
  __shared__ int32_t s_scan[8];
  __shared__ int64_t s_range[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  // tiles before sequence b and in total (same clamped lengths as the decode kernel)
  const int chunk = (n_seq + 255) / 256;
  const int lo = min(tid * chunk, n_seq), hi = min(lo + chunk, n_seq);
  int before = 0, all = 0;
  for (int i = lo; i < hi; ++i) {
    const int32_t L = min(max(seqlens[i], 0), lay.max_len);
    const int nt = (L + lay.tile - 1) / lay.tile;
    all += nt;
    if (i < b) before += nt;
  }
  for (int off = 32; off > 0; off >>= 1) {
    before += __shfl_xor(before, off, 64);
    all += __shfl_xor(all, off, 64);
  }
  if (lane == 0) {
    s_scan[wave] = before;
    s_scan[4 + wave] = all;
  }
  __syncthreads();
  if (tid == 0) {
    const int64_t start = (int64_t)s_scan[0] + s_scan[1] + s_scan[2] + s_scan[3];
    const int64_t total = (int64_t)s_scan[4] + s_scan[5] + s_scan[6] + s_scan[7];
    const int32_t L = min(max(seqlens[b], 0), lay.max_len);
    const int64_t nb = (L + lay.tile - 1) / lay.tile;
    int64_t wf = 0, wl = 0;
    if (nb > 0) {
      wf = unit_of_tile(start, total, lay.n_splits);
      wl = unit_of_tile(start + nb - 1, total, lay.n_splits);
    }
    s_range[0] = wf;
    s_range[1] = (nb == 0 || wf == wl) ? 0 : wl - wf + 1;   // 0: the decode kernel wrote this sequence
    s_range[2] = total;
  }
  __syncthreads();
  const int64_t wf = s_range[0], count = s_range[1], total = s_range[2];
  if (count == 0) return;
  const int r = blockIdx.y * kRowsPerBlock + (tid >> 4);
  if (r >= rows_per_seq) return;
  const int d0 = (tid & 15) * 32;

  // Online merge over the pieces, four at a time: the stats and the 32 values
  // of all four pieces are loaded before any is used (one memory latency per
  // group), then folded in against a running maximum m:
  //   acc <- acc 2^(m - m') + 2^(m_k - m') O_k,  tot likewise with l_k.
  float m = -INFINITY, tot = 0.f;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  for (int64_t k0 = 0; k0 < count; k0 += kGroup) {
    float sm[kGroup], sl[kGroup];
    f32x4 v[kGroup][8];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int64_t w = wf + min(k0 + j, count - 1);   // clamped: a repeated piece is masked below
      const float* st = ws_stats + ((w + b) * rows_per_seq + r) * 2;
      sm[j] = st[0];
      sl[j] = st[1];
      const f32x4* src = (const f32x4*)(ws_o + ((w + b) * rows_per_seq + r) * kDc + d0);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = src[i];
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int64_t w = wf + k0 + j;
      if (k0 + j >= count) break;
      // a unit that owns no tile left nothing in its slot
      if (unit_first_tile(w, total, lay.n_splits) == unit_first_tile(w + 1, total, lay.n_splits)) continue;
      if (!(sl[j] > 0.f)) continue;
      const float mn = fmaxf(m, sm[j]);
      const float keep = exp2f(m - mn);          // 0 while nothing is accumulated (m = -inf)
      const float wgt = exp2f(sm[j] - mn);
      tot = fmaf(tot, keep, wgt * sl[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * i + e] = fmaf(acc[4 * i + e], keep, wgt * v[j][i][e]);
      m = mn;
    }
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  u32x4* dst = (u32x4*)(o_lat + ((int64_t)b * rows_per_seq + r) * kDc + d0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (uint32_t)f32_to_bf16_bits(acc[8 * i + 2 * e] * inv) |
             ((uint32_t)f32_to_bf16_bits(acc[8 * i + 2 * e + 1] * inv) << 16);
    dst[i] = v;
  }
  if ((tid & 15) == 0)
    lse[(int64_t)b * rows_per_seq + r] = tot > 0.f ? (m + log2f(tot)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

mla_status launch_combine_stream(const mla_dims& d, const DecodePlan& plan, int32_t n_seq, int32_t q_per_seq,
                                 const int32_t* seqlens, const void* ws, void* o_lat, float* lse, hipStream_t st) {
  const int rows = q_per_seq * d.n_heads;
  const float* ws_o = static_cast<const float*>(ws);
  const float* ws_stats = ws_o + plan.ws_stats_offset_floats;
  dim3 grid(n_seq, (rows + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(combine_stream_kernel, grid, dim3(256), 0, st, ws_o, ws_stats, seqlens, n_seq, rows,
                     plan.layout, static_cast<uint16_t*>(o_lat), lse);
  return launch_status();
}

}  // namespace mla
