// Tuned gfx950 kernels for the two per-head projections around the latent
// attention (bf16 in, fp32 accumulation on MFMA 32x32x16, bf16 out):
//   absorb:  q_abs[t,s,:d_c] = W_UK[s]^T q_nope[t,s]  (+ RoPE of q_R into q_abs[t,s,d_c:])
//   up-proj: out[t,s,:]      = W_UV[s] o_lat[t,s]
// Both are computed transposed (output rows = feature, columns = tokens) so
// that the 32 tokens of a block land in the 32 lanes and each lane writes 4
// consecutive features.  Both are weight-streaming (a decode step has few
// tokens), so the contraction sizes are compile-time constants: every loop
// unrolls and each wave issues all of its global loads before the first MFMA
// waits on one, instead of paying one memory latency per k-step.
//  * absorb: W_UK[s] is stored [d_nope][d_c] (feature-contiguous); a
//    [d_nope x 128] slab is staged in LDS and read back with the LDS
//    transpose read, which yields 4 consecutive contraction elements per lane.
//  * up-proj: W_UV[s] is stored [d_v][d_c], i.e. contraction-contiguous, so
//    both MFMA operands come straight from global memory (16 bytes per lane).
//    The contraction is split over the 4 waves (128 latent dims each) and the
//    four fp32 partial tiles are summed through LDS.
#include <math.h>

#include "append_body.h"
#include "decode_latent576.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) float lds_f32;

constexpr int kAbsorbCols = 128;       // latent columns per absorb work-group
constexpr int kNope = 128;             // d_nope of the tuned absorb
constexpr int kUpDc = 512;             // d_c of the tuned up-projection
constexpr int kUpDv = 128;             // d_v of the tuned up-projection

__device__ __forceinline__ int swz8(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// 4 fp32 -> 4 bf16 (round to nearest even) packed in 8 bytes
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
  u32x2 r;
  r[0] = (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
  r[1] = (uint32_t)f32_to_bf16_bits(c) | ((uint32_t)f32_to_bf16_bits(d) << 16);
  return r;
}

// grid (H, d_c / 128), block 256.  LDS slab row n (one contraction index) holds
// latent columns cblk*128 .. +127 as 16 chunks of 16 bytes; chunk c of row n is
// stored at chunk (c & ~7) | ((c ^ swz8(n)) & 7) so the transpose reads (4 rows
// x 32 bytes per 16 lanes) are free of bank conflicts.  Wave w computes latent
// columns 32w .. 32w+31 of the block for every 32-token block in turn; the
// next block's query fragments are loaded while the current one is multiplied.
struct AbsorbArgs {
  const uint16_t* q_nope;
  const uint16_t* q_rope;
  const int32_t* pos;
  const uint16_t* w_uk;
  uint16_t* q_abs;
  int n_tok, H, d_c, d_rope;
};

// The absorb of head s, latent columns cblk*128 .. +127 (ny = d_c / 128 blocks per head).
__device__ __forceinline__ void absorb_body(const AbsorbArgs& aa, int s, int cblk, int ny, const RopeFreqs& freqs) {
  const uint16_t* __restrict__ q_nope = aa.q_nope;
  const uint16_t* __restrict__ q_rope = aa.q_rope;
  const int32_t* __restrict__ pos = aa.pos;
  const uint16_t* __restrict__ w_uk = aa.w_uk;
  uint16_t* __restrict__ q_abs = aa.q_abs;
  const int n_tok = aa.n_tok, H = aa.H, d_c = aa.d_c, d_rope = aa.d_rope;
  constexpr int kSteps = kNope / 16;                 // 8 k-steps of 16
  constexpr int kChunks = kNope * 16 / 256;          // slab chunks per thread
  __shared__ __attribute__((aligned(16))) uint8_t slab_raw[kNope * kAbsorbCols * 2];
  lds_u8* slab = (lds_u8*)slab_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d_k = d_c + d_rope;
  const int gi = lane >> 4, sp = lane & 15, half = lane >> 5;

  // The rotated query part of head s is shared by its d_c / 128 work-groups
  // (work-group cblk takes tokens t = cblk mod gridDim.y).  The inputs of this
  // thread's first two rotations are loaded before the slab, so that the fp64
  // cos/sin run while the slab loads are in flight (loads complete in order).
  const int pairs = d_rope / 2;
  const int n_rope = ((n_tok - cblk + ny - 1) / ny) * pairs;
  auto rope_item = [&](int i, int* t, int* p) {   // only called with pairs > 0
    *t = cblk + ny * (i / pairs);
    *p = i % pairs;
  };
  // (indices clamped so the loads need no branch; unused ones are dropped below).
  // Without a RoPE part (d_rope = 0) q_rope and pos may be null and nothing is read.
  int32_t r_pos[2] = {0, 0};
  uint32_t r_q[2] = {0u, 0u};
  double r_f[2] = {0.0, 0.0};
  if (pairs > 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int t, p;
      rope_item(min(tid + 256 * j, max(n_rope - 1, 0)), &t, &p);
      t = min(t, n_tok - 1);
      r_pos[j] = pos[t];
      r_q[j] = *(const uint32_t*)(q_rope + ((int64_t)t * H + s) * d_rope + 2 * p);
      r_f[j] = freqs.inv_freq[p];
    }
  }
  // slab loads (W_UK[s][:, cblk*128 .. +127]) and the first block's queries, all in flight together
  const uint16_t* wsrc = w_uk + (int64_t)s * kNope * d_c + cblk * kAbsorbCols;
  u32x4 wv[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int idx = tid + 256 * i, n = idx >> 4, c = idx & 15;
    wv[i] = *(const u32x4*)(wsrc + (int64_t)n * d_c + c * 8);
  }
  auto load_q = [&](int t0, bf16x8 (&qf)[kSteps]) {
    const int t = min(t0 + (lane & 31), n_tok - 1);
    const bf16x8* qsrc = (const bf16x8*)(q_nope + ((int64_t)t * H + s) * kNope) + half;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) qf[ks] = qsrc[2 * ks];
  };
  bf16x8 qf[kSteps];
  load_q(0, qf);
  auto rotate = [&](int32_t pt, uint32_t qv, double f) {
    float cs, sn, ox, oy;
    rope_cos_sin(pt, f, &cs, &sn);
    rope_pair(bf16_bits_to_f32((uint16_t)(qv & 0xffffu)), bf16_bits_to_f32((uint16_t)(qv >> 16)), cs, sn, &ox, &oy);
    return (uint32_t)f32_to_bf16_bits(ox) | ((uint32_t)f32_to_bf16_bits(oy) << 16);
  };
  auto rope_dst = [&](int i) {
    int t, p;
    rope_item(i, &t, &p);
    return (uint32_t*)(q_abs + ((int64_t)t * H + s) * d_k + d_c + 2 * p);
  };
  // computed for every lane (clamped items included) so the preloads stay ahead of the slab
  if (pairs > 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t v = rotate(r_pos[j], r_q[j], r_f[j]);
      if (tid + 256 * j < n_rope) *rope_dst(tid + 256 * j) = v;
    }
    for (int i = tid + 512; i < n_rope; i += 256) {   // more than 512 rotations: rest loaded here
      int t, p;
      rope_item(i, &t, &p);
      *rope_dst(i) = rotate(pos[t], *(const uint32_t*)(q_rope + ((int64_t)t * H + s) * d_rope + 2 * p), freqs.inv_freq[p]);
    }
  }
  // the first block's queries are consumed here, together with the slab, so
  // that both sets of loads share one memory latency
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) asm volatile("" ::"v"(qf[ks]));
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int idx = tid + 256 * i, n = idx >> 4, c = idx & 15;
    const int pc = (c & ~7) | ((c ^ swz8(n)) & 7);
    *(lds_u32x4*)(slab + n * 256 + pc * 16) = wv[i];
  }
  __syncthreads();

  // per-lane transpose-read offsets for k-step 0 (k-step ks adds 16 rows = 4 KB)
  uint32_t tr_off[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int n = 8 * (gi >> 1) + 4 * hh + (sp >> 2);
    const int col = 32 * wave + 16 * (gi & 1) + 4 * (sp & 3);
    const int c = col >> 3;
    const int pc = (c & ~7) | ((c ^ swz8(n)) & 7);
    tr_off[hh] = (uint32_t)(uintptr_t)slab + n * 256 + pc * 16 + (col & 7) * 2;
  }
  for (int t0 = 0; t0 < n_tok; t0 += 32) {
    bf16x8 qn[kSteps];
    if (t0 + 32 < n_tok) load_q(t0 + 32, qn);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)(tr_off[0] + ks * 16 * 256));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)(tr_off[1] + ks * 16 * 256));
      const bf16x8 a = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], acc, 0, 0, 0);
    }
    const int t = t0 + (lane & 31);
    if (t < n_tok) {
      uint16_t* dst = q_abs + ((int64_t)t * H + s) * d_k + cblk * kAbsorbCols + 32 * wave + 4 * half;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(u32x2*)(dst + 8 * g) = pack4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
    }
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) qf[ks] = qn[ks];
  }
}

__global__ void __launch_bounds__(256) absorb_tuned_kernel(AbsorbArgs aa, RopeFreqs freqs) {
  absorb_body(aa, blockIdx.x, blockIdx.y, gridDim.y, freqs);
}

struct AppendArgs {
  const uint16_t* c_kv;
  const uint16_t* k_rope;
  const int32_t* seq_id;
  const int32_t* pos;
  const int32_t* block_table;
  uint8_t* pool;
  int64_t n_pool_blocks, block_bytes;
  int n_seq, max_blocks, block_size, d_c, d_rope;
};

// One launch for the two independent head-of-step calls: work-groups 0 ..
// H ny - 1 absorb (head b / ny, latent block b % ny), the rest append one new
// token each.  The appends are short and fill the CUs the absorb leaves idle.
template <bool kFp8>
__global__ void __launch_bounds__(256) absorb_append_kernel(AbsorbArgs aa, AppendArgs pa, int ny, RopeFreqs freqs) {
  __shared__ float red[256];
  const int n_abs = aa.H * ny;
  const int b = blockIdx.x;
  if (b < n_abs) {
    absorb_body(aa, b / ny, b % ny, ny, freqs);
  } else {
    append_token<uint16_t, kFp8>(b - n_abs, pa.c_kv, pa.k_rope, pa.seq_id, pa.pos, pa.block_table, pa.n_seq,
                                 pa.max_blocks, pa.pool, pa.n_pool_blocks, pa.block_bytes, pa.block_size, pa.d_c,
                                 pa.d_rope, freqs, red);
  }
}

// grid (H, ceil(n_tok / 32)), block 256.  Wave w contracts latent dims
// 128w .. 128w+127 for all d_v/32 output-row blocks of the block's 32 tokens
// (all its operands are loaded up front), writes its fp32 partial tiles to
// LDS, and after the barrier finishes output-row block w by summing the four
// partials in a fixed order.  kGate: the fp32 result is multiplied by
// sigmoid(gate) of the same element before its one rounding to bf16.
template <bool kGate>
__global__ void __launch_bounds__(256) up_proj_tuned_kernel(const uint16_t* __restrict__ o_lat,
                                                            const uint16_t* __restrict__ w_uv,
                                                            const uint16_t* __restrict__ gate,
                                                            uint16_t* __restrict__ out, int n_tok, int H) {
  constexpr int kVb = kUpDv / 32;                    // 4 output-row blocks
  constexpr int kSlice = kUpDc / 4;                  // latent dims per wave
  constexpr int kSteps = kSlice / 16;                // 8 k-steps
  static_assert(kVb == 4, "one output-row block per wave in the reduction");
  __shared__ __attribute__((aligned(16))) float red_raw[4 * kVb * 16 * 64];   // [wave][vb][reg][lane]
  lds_f32* red = (lds_f32*)red_raw;
  const int s = blockIdx.x;
  const int t0 = blockIdx.y * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int t = t0 + (lane & 31);
  const int tc = min(t, n_tok - 1);
  const bf16x8* bsrc = (const bf16x8*)(o_lat + ((int64_t)tc * H + s) * kUpDc + kSlice * wave) + half;
  bf16x8 bf[kSteps];
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks) bf[ks] = bsrc[2 * ks];
  // this lane's gate logits: output rows 32 w + 8 g + 4 half .. +3 of token t
  u32x2 graw[4];
  if constexpr (kGate) {
    const uint16_t* gsrc = gate + ((int64_t)tc * H + s) * kUpDv + 32 * wave + 4 * half;
#pragma unroll
    for (int g = 0; g < 4; ++g) graw[g] = *(const u32x2*)(gsrc + 8 * g);
  }
  bf16x8 af[kVb][kSteps];
#pragma unroll
  for (int vb = 0; vb < kVb; ++vb) {
    const bf16x8* asrc = (const bf16x8*)(w_uv + ((int64_t)s * kUpDv + 32 * vb + (lane & 31)) * kUpDc + kSlice * wave) + half;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) af[vb][ks] = asrc[2 * ks];
  }
  __builtin_amdgcn_sched_barrier(0);   // every load is issued before the first MFMA waits
  f32x16 acc[kVb];
#pragma unroll
  for (int vb = 0; vb < kVb; ++vb) acc[vb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
    for (int vb = 0; vb < kVb; ++vb) acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[vb][ks], bf[ks], acc[vb], 0, 0, 0);
#pragma unroll
  for (int vb = 0; vb < kVb; ++vb)
#pragma unroll
    for (int i = 0; i < 16; ++i) red[((wave * kVb + vb) * 16 + i) * 64 + lane] = acc[vb][i];
  __syncthreads();
  // output-row block vb = wave: rows 32*vb + 8(i/4) + 4*half + i%4, token t
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = red[((0 * kVb + wave) * 16 + i) * 64 + lane];
#pragma unroll
    for (int w2 = 1; w2 < 4; ++w2) x += red[((w2 * kVb + wave) * 16 + i) * 64 + lane];
    v[i] = x;
  }
  if constexpr (kGate) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w2 = graw[g][e >> 1];
        v[4 * g + e] *= sigmoid_f32(__uint_as_float((e & 1) ? (w2 & 0xffff0000u) : (w2 << 16)));
      }
  }
  if (t < n_tok) {
    uint16_t* dst = out + ((int64_t)t * H + s) * kUpDv + 32 * wave + 4 * half;
#pragma unroll
    for (int g = 0; g < 4; ++g) *(u32x2*)(dst + 8 * g) = pack4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
  }
}

}  // namespace

bool absorb_tuned_applies(const mla_dims& d) {
  return d.act_dtype == MLA_BF16 && d.d_c % kAbsorbCols == 0 && d.d_nope == kNope && d.d_rope % 2 == 0;
}

mla_status launch_absorb_tuned(const mla_dims& d, int32_t n_tok, const void* q_nope, const void* q_rope,
                               const int32_t* pos, const void* w_uk, void* q_abs, hipStream_t st) {
  const RopeFreqs f = make_rope_freqs(d);
  dim3 grid(d.n_heads, d.d_c / kAbsorbCols);
  const AbsorbArgs aa{static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope), pos,
                      static_cast<const uint16_t*>(w_uk), static_cast<uint16_t*>(q_abs), n_tok, d.n_heads, d.d_c,
                      d.d_rope};
  hipLaunchKernelGGL(absorb_tuned_kernel, grid, dim3(256), 0, st, aa, f);
  return launch_status();
}

mla_status launch_absorb_append(const mla_dims& d, int32_t n_q, const void* q_nope, const void* q_rope,
                                const int32_t* q_pos, const void* w_uk, void* q_abs, int32_t n_kv, const void* c_kv,
                                const void* k_rope, const int32_t* seq_id, const int32_t* pos,
                                const int32_t* block_table, int32_t n_seq, int32_t max_blocks, void* pool,
                                int64_t n_pool_blocks, hipStream_t st) {
  const RopeFreqs f = make_rope_freqs(d);
  const int ny = d.d_c / kAbsorbCols;
  const AbsorbArgs aa{static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope), q_pos,
                      static_cast<const uint16_t*>(w_uk), static_cast<uint16_t*>(q_abs), n_q, d.n_heads, d.d_c,
                      d.d_rope};
  const AppendArgs pa{static_cast<const uint16_t*>(c_kv), static_cast<const uint16_t*>(k_rope), seq_id, pos,
                      block_table, static_cast<uint8_t*>(pool), n_pool_blocks,
                      static_cast<int64_t>(mla_cache_block_bytes(&d)), n_seq, max_blocks, d.block_size, d.d_c,
                      d.d_rope};
  const dim3 grid((unsigned)(d.n_heads * ny + n_kv));
  if (d.cache_dtype == MLA_FP8_E4M3)
    hipLaunchKernelGGL(absorb_append_kernel<true>, grid, dim3(256), 0, st, aa, pa, ny, f);
  else
    hipLaunchKernelGGL(absorb_append_kernel<false>, grid, dim3(256), 0, st, aa, pa, ny, f);
  return launch_status();
}

bool up_proj_tuned_applies(const mla_dims& d) {
  return d.act_dtype == MLA_BF16 && d.d_c == kUpDc && d.d_v == kUpDv;
}

mla_status launch_up_proj_tuned(const mla_dims& d, int32_t n_tok, const void* o_lat, const void* w_uv,
                                const void* gate, void* out, hipStream_t st) {
  dim3 grid(d.n_heads, (n_tok + 31) / 32);
  if (gate)
    hipLaunchKernelGGL(up_proj_tuned_kernel<true>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(o_lat),
                       static_cast<const uint16_t*>(w_uv), static_cast<const uint16_t*>(gate),
                       static_cast<uint16_t*>(out), n_tok, d.n_heads);
  else
    hipLaunchKernelGGL(up_proj_tuned_kernel<false>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(o_lat),
                       static_cast<const uint16_t*>(w_uv), nullptr, static_cast<uint16_t*>(out), n_tok, d.n_heads);
  return launch_status();
}

}  // namespace mla
