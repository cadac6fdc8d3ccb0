// The projections upstream of the latent attention ("DeepSeek-V3 解读：
// Multi-head Latent Attention", MLA：高层次的思路 and 为什么需要解耦 RoPE):
//   c_Q = W_DQ h,  c_KV = W_DKV h,  k_R = W_KR h        (one GEMM: W_down = [W_DQ; W_DKV; W_KR])
//   [q_C | q_R] = W_UQ[s] c_Q per head                   (one GEMM over all heads)
// Each projection is an activation and is rounded once to bf16 before it is
// used; the latent and the shared key then go through the append kernel
// (RoPE, cache dtype, paging) and the query parts through the absorb kernel,
// so the fused calls produce exactly what projecting and then calling
// mla_append_cache / mla_absorb_q would.
//
// W_UK is not pre-composed into W_UQ: the composed map W_UK[s]^T W_UQ[s] is a
// d_c x d_cq matrix per head (512 x 1536 at DeepSeek-V3 shape, 1.5 MB), three
// times the bytes of the two factors it replaces (W_UQ's 128 x 1536 rows and
// W_UK[s]'s 128 x 512), and at decode the weights are what is read.
//
// The GEMM Y = X W^T (X [n_tok][K] tokens, W [N][K] weights, both bf16 and
// contraction-contiguous) is computed transposed on MFMA 32x32x16: each
// work-group owns 64 output features x 64 tokens and a range of the
// contraction (split-K, so that a few tokens still spread the weight stream
// over the whole chip); its four waves take a quarter of that range each,
// with both operands read straight from global memory, 16 bytes per lane, 8
// k-steps of loads issued before their MFMAs.  The four partial tiles are
// summed through LDS and each split writes an fp32 partial [split][n_tok][N];
// the small epilogue kernels sum the splits in a fixed order.  (32 features
// per work-group, or 16 k-steps per batch, measured slower at 64 tokens.)
#include <algorithm>

#include "decode_latent576.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

#ifndef GEMM_FT
#define GEMM_FT 2
#endif
#ifndef GEMM_STEPS
#define GEMM_STEPS 8
#endif
constexpr int kGemmTok = 64;            // tokens per work-group (two MFMA column tiles)
constexpr int kFT = GEMM_FT;            // 32-feature tiles per work-group
constexpr int kGemmFeat = 32 * kFT;     // features per work-group
constexpr int kGemmSteps = GEMM_STEPS;  // k-steps (16 each) loaded per wave before its MFMAs
constexpr int kRedPitch = kGemmFeat + 4;   // LDS floats per token row of a wave's partial tile (padded)

// grid (ceil(N / kGemmFeat), ceil(n_tok / 64), S), block 256.
__global__ void __launch_bounds__(256) xwt_gemm_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                       int n_tok, int N, int K, int steps_per_split,
                                                       float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float red_raw[4 * kGemmTok * kRedPitch];
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int f0 = blockIdx.x * kGemmFeat, t0 = blockIdx.y * kGemmTok, z = blockIdx.z;
  const int ksteps = K / 16;
  const int z0 = z * steps_per_split, z1 = min(z0 + steps_per_split, ksteps);
  const int per = (z1 - z0 + 3) / 4;
  const int w0 = min(z0 + wave * per, z1), w1 = min(w0 + per, z1);

  // A: feature rows f0 + 32 ft + lane % 32; B: token rows t0 + 32 tt + lane % 32 (clamped; out-of-range rows are
  // not stored)
  const bf16x8* arow[kFT];
#pragma unroll
  for (int ft = 0; ft < kFT; ++ft) arow[ft] = (const bf16x8*)(W + (int64_t)min(f0 + 32 * ft + (lane & 31), N - 1) * K) + half;
  const bf16x8* brow[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) brow[tt] = (const bf16x8*)(X + (int64_t)min(t0 + 32 * tt + (lane & 31), n_tok - 1) * K) + half;

  f32x16 acc[kFT][2];
#pragma unroll
  for (int ft = 0; ft < kFT; ++ft) acc[ft][0] = acc[ft][1] = f32x16{};
  for (int ks = w0; ks < w1; ks += kGemmSteps) {
    bf16x8 a[kGemmSteps][kFT], b[kGemmSteps][2];
#pragma unroll
    for (int j = 0; j < kGemmSteps; ++j) {
      const int k = min(ks + j, w1 - 1);
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) a[j][ft] = arow[ft][2 * k];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) b[j][tt] = brow[tt][2 * k];
    }
#pragma unroll
    for (int j = 0; j < kGemmSteps; ++j)
      if (ks + j < w1) {
#pragma unroll
        for (int ft = 0; ft < kFT; ++ft)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            acc[ft][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j][ft], b[j][tt], acc[ft][tt], 0, 0, 0);
      }
  }

  // lane holds token 32 tt + lane % 32, features 32 ft + 8 g + 4 half + 0..3 (g = i / 4)
  lds_f32x4* red = (lds_f32x4*)(__attribute__((address_space(3))) float*)red_raw;
#pragma unroll
  for (int ft = 0; ft < kFT; ++ft)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = wave * kGemmTok + 32 * tt + (lane & 31);
        red[(row * kRedPitch + 32 * ft + 8 * g + 4 * half) / 4] =
            f32x4{acc[ft][tt][4 * g], acc[ft][tt][4 * g + 1], acc[ft][tt][4 * g + 2], acc[ft][tt][4 * g + 3]};
      }
  __syncthreads();
  // thread: token r = tid / 4, features 8 (tid % 4) + 32 ft .. +7, summed over the waves in order
  const int r = tid >> 2, t = t0 + r;
#pragma unroll
  for (int ft = 0; ft < kFT; ++ft) {
    const int c8 = 32 * ft + 8 * (tid & 3);
    f32x4 s0 = red[(r * kRedPitch + c8) / 4], s1 = red[(r * kRedPitch + c8 + 4) / 4];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      s0 += red[((w * kGemmTok + r) * kRedPitch + c8) / 4];
      s1 += red[((w * kGemmTok + r) * kRedPitch + c8 + 4) / 4];
    }
    if (t < n_tok) {
      float* dst = part + ((int64_t)z * n_tok + t) * N + f0 + c8;
      if (f0 + c8 + 4 <= N) *(f32x4*)dst = s0;
      if (f0 + c8 + 8 <= N) *(f32x4*)(dst + 4) = s1;
    }
  }
}

// Epilogues: grid (ceil(N / 1024), n_tok), block 256; thread i of a work-group
// takes features 4i .. 4i+3 of the block's 1024 (the segment boundaries below
// are multiples of 4): the sum of the S partials in split order, rounded to bf16.
__device__ __forceinline__ bool sum_partials4(const float* __restrict__ part, int S, int n_tok, int N, int t, int n,
                                              u32x2* out) {
  if (n >= N) return false;
  f32x4 v = *(const f32x4*)(part + (int64_t)t * N + n);
  for (int z = 1; z < S; ++z) v += *(const f32x4*)(part + ((int64_t)z * n_tok + t) * N + n);
  (*out)[0] = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
  (*out)[1] = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
  return true;
}

// Down-projection: features [0, d_cq) are c_q [n_tok][d_cq], [d_cq, d_cq + d_c)
// the latent [n_tok][d_c] and the rest the raw shared key [n_tok][d_rope]
// (workspace, for the append kernel).
__global__ void __launch_bounds__(256) down_reduce_kernel(const float* __restrict__ part, int S, int n_tok, int N,
                                                          int d_cq, int d_c, uint16_t* __restrict__ c_q,
                                                          uint16_t* __restrict__ c_kv, uint16_t* __restrict__ k_rope) {
  const int t = blockIdx.y, n = 1024 * blockIdx.x + 4 * threadIdx.x;
  const int d_rope = N - d_cq - d_c;
  u32x2 b;
  if (!sum_partials4(part, S, n_tok, N, t, n, &b)) return;
  uint16_t* dst = n < d_cq ? c_q + (int64_t)t * d_cq + n
                  : n < d_cq + d_c ? c_kv + (int64_t)t * d_c + (n - d_cq)
                                   : k_rope + (int64_t)t * d_rope + (n - d_cq - d_c);
  *(u32x2*)dst = b;
}

// Query up-projection: feature n = s (d_nope + d_rope) + r is q_C[t, s, r]
// (r < d_nope) or the raw q_R[t, s, r - d_nope].
__global__ void __launch_bounds__(256) q_split_kernel(const float* __restrict__ part, int S, int n_tok, int H,
                                                      int d_nope, int d_rope, uint16_t* __restrict__ q_nope,
                                                      uint16_t* __restrict__ q_rope) {
  const int t = blockIdx.y, n = 1024 * blockIdx.x + 4 * threadIdx.x;
  const int dq = d_nope + d_rope;
  u32x2 b;
  if (!sum_partials4(part, S, n_tok, H * dq, t, n, &b)) return;
  const int s = n / dq, r = n % dq;
  uint16_t* dst = r < d_nope ? q_nope + ((int64_t)t * H + s) * d_nope + r
                             : q_rope + ((int64_t)t * H + s) * d_rope + (r - d_nope);
  *(u32x2*)dst = b;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Split count: about 512 work-groups (two per CU) whatever the token count,
// at least 4 k-steps per wave.  A function of the shape only, so that the
// workspace size does not depend on the device.
int gemm_splits(int64_t n_tok, int64_t N, int64_t K) {
  const int64_t tiles = ((N + kGemmFeat - 1) / kGemmFeat) * ((n_tok + kGemmTok - 1) / kGemmTok);
  const int64_t ksteps = K / 16;
  int64_t s = (512 + tiles - 1) / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(1, ksteps / 16));
  return (int)std::max<int64_t>(s, 1);
}

void launch_gemm(const uint16_t* X, const uint16_t* W, int n_tok, int N, int K, int S, float* part, hipStream_t st) {
  const int ksteps = K / 16;
  const int steps_per_split = (ksteps + S - 1) / S;
  dim3 grid((N + kGemmFeat - 1) / kGemmFeat, (n_tok + kGemmTok - 1) / kGemmTok, S);
  hipLaunchKernelGGL(xwt_gemm_kernel, grid, dim3(256), 0, st, X, W, n_tok, N, K, steps_per_split, part);
}

}  // namespace

size_t project_down_workspace_bytes(const mla_dims& d, int64_t n_tok, int64_t d_model, int64_t d_cq) {
  const int64_t N = d_cq + d.d_c + d.d_rope;
  const int S = gemm_splits(n_tok, N, d_model);
  return up256((size_t)S * n_tok * N * 4) + up256((size_t)n_tok * d.d_c * 2) + up256((size_t)n_tok * d.d_rope * 2);
}

mla_status launch_project_down(const mla_dims& d, int32_t n_tok, int32_t d_model, int32_t d_cq, const void* h,
                               const void* w_down, const int32_t* seq_id, const int32_t* pos,
                               const int32_t* block_table, int32_t n_seq, int32_t max_blocks, void* pool,
                               int64_t n_pool_blocks, void* c_q, void* ws, hipStream_t st) {
  const int N = d_cq + d.d_c + d.d_rope;
  const int S = gemm_splits(n_tok, N, d_model);
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* part = reinterpret_cast<float*>(p);
  p += up256((size_t)S * n_tok * N * 4);
  uint16_t* ckv = reinterpret_cast<uint16_t*>(p);
  p += up256((size_t)n_tok * d.d_c * 2);
  uint16_t* kr = reinterpret_cast<uint16_t*>(p);
  launch_gemm(static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_down), n_tok, N, d_model, S, part, st);
  hipLaunchKernelGGL(down_reduce_kernel, dim3((N + 1023) / 1024, n_tok), dim3(256), 0, st, part, S, n_tok, N, d_cq, d.d_c,
                     static_cast<uint16_t*>(c_q), ckv, kr);
  const mla_status s = launch_status();
  if (s != MLA_OK) return s;
  return launch_append_generic(d, n_tok, ckv, kr, seq_id, pos, block_table, n_seq, max_blocks, pool, n_pool_blocks,
                               st);
}

size_t absorb_from_latent_workspace_bytes(const mla_dims& d, int64_t n_tok, int64_t d_cq) {
  const int64_t N = (int64_t)d.n_heads * (d.d_nope + d.d_rope);
  const int S = gemm_splits(n_tok, N, d_cq);
  return up256((size_t)S * n_tok * N * 4) + up256((size_t)n_tok * d.n_heads * d.d_nope * 2) +
         up256((size_t)n_tok * d.n_heads * d.d_rope * 2);
}

mla_status launch_absorb_from_latent(const mla_dims& d, int32_t n_tok, int32_t d_cq, const void* c_q,
                                     const void* w_uq, const int32_t* pos, const void* w_uk, void* q_abs, void* ws,
                                     hipStream_t st) {
  const int N = d.n_heads * (d.d_nope + d.d_rope);
  const int S = gemm_splits(n_tok, N, d_cq);
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* part = reinterpret_cast<float*>(p);
  p += up256((size_t)S * n_tok * N * 4);
  uint16_t* qn = reinterpret_cast<uint16_t*>(p);
  p += up256((size_t)n_tok * d.n_heads * d.d_nope * 2);
  uint16_t* qr = reinterpret_cast<uint16_t*>(p);
  launch_gemm(static_cast<const uint16_t*>(c_q), static_cast<const uint16_t*>(w_uq), n_tok, N, d_cq, S, part, st);
  hipLaunchKernelGGL(q_split_kernel, dim3((N + 1023) / 1024, n_tok), dim3(256), 0, st, part, S, n_tok, d.n_heads,
                     d.d_nope, d.d_rope,
                     qn, qr);
  const mla_status s = launch_status();
  if (s != MLA_OK) return s;
  if (absorb_tuned_applies(d) && ((uintptr_t)w_uk & 15) == 0 && ((uintptr_t)q_abs & 15) == 0)
    return launch_absorb_tuned(d, n_tok, qn, qr, pos, w_uk, q_abs, st);
  return launch_absorb_generic(d, n_tok, qn, qr, pos, w_uk, q_abs, st);
}

}  // namespace mla
