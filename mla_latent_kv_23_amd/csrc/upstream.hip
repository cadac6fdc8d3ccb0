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
// over the whole chip).  Both operands are staged through LDS in stages of
// 128 contraction elements, loaded as whole 256-byte row segments (16 lanes
// per row), two stages in flight in registers; each wave multiplies one
// 32 x 32 output tile out of LDS.  Each split writes an fp32 partial
// [split][n_tok][N]; the small epilogue kernels sum the splits in a fixed
// order.  (Reading the MFMA fragments straight from global memory touches 32
// bytes of 32 rows per load instruction and measured 1.5-2x slower.)
#include <algorithm>

#include "decode_latent576.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr int kGemmTok = 64;            // tokens per work-group (two MFMA column tiles)
constexpr int kGemmFeat = 64;           // features per work-group (two MFMA row tiles)
constexpr int kChunkSteps = 8;          // k-steps (16 contraction elements each) per LDS stage (4 and 16 measured slower)
constexpr int kChunkK = 16 * kChunkSteps;
constexpr int kParts = 2 * kChunkSteps; // 16-byte parts per staged row
constexpr int kRowB = kChunkK * 2 + 16; // LDS bytes per staged row (padded: conflict-free fragment reads)
constexpr int kStageB = (kGemmFeat + kGemmTok) * kRowB;
constexpr int kPieces = (kGemmFeat + kGemmTok) * kParts / 256;   // 16-byte loads per thread per stage

// Where a split's result goes: fp32 partials part[split][n_tok][N], or (a
// single split) bf16 straight into the query parts: feature n = s (d_nope +
// d_rope) + r is q_nope[t, s, r] (r < d_nope) or q_rope[t, s, r - d_nope].
struct GemmOut {
  float* part;
  uint16_t *q_nope, *q_rope;
  int d_nope, d_rope;
};

// grid (ceil(N / 64), ceil(n_tok / 64), S), block 256.  Each stage holds 128
// contraction elements of the 64 weight rows and the 64 token rows; thread t
// loads pieces p = t + 256 j: row p / 16, 16-byte part p % 16 (16 consecutive
// lanes read one 256-byte row segment).  Two stages are in flight in
// registers while the previous one is multiplied out of LDS.  Wave w computes
// the 32 x 32 output tile (features 32 (w % 2), tokens 32 (w / 2)).
__global__ void __launch_bounds__(256) xwt_gemm_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                       int n_tok, int N, int K, int steps_per_split, GemmOut go) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[2 * kStageB];
  lds_u8* lds = (lds_u8*)lds_raw;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ft = wave & 1, tt = wave >> 1;
  const int f0 = blockIdx.x * kGemmFeat, t0 = blockIdx.y * kGemmTok, z = blockIdx.z;
  const int ksteps = K / 16;
  const int ks0 = z * steps_per_split, ks1 = min(ks0 + steps_per_split, ksteps);
  const int n_chunks = (ks1 - ks0 + kChunkSteps - 1) / kChunkSteps;

  // this thread's source rows (clamped: rows past N or n_tok are loaded but never stored)
  const uint16_t* src[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const int p = tid + 256 * j, row = p / kParts, part = p % kParts;
    const uint16_t* base = row < kGemmFeat ? W + (int64_t)min(f0 + row, N - 1) * K
                                           : X + (int64_t)min(t0 + row - kGemmFeat, n_tok - 1) * K;
    src[j] = base + 16 * ks0 + 8 * part;
  }
  // k-steps past the split's end read the split's last k-step (in bounds) and are skipped by the MFMAs
  auto load = [&](u32x4 (&r)[kPieces], int c) {
    const int kk = (tid % kParts) >> 1;   // this thread's k-step in the stage (the same for every piece)
    const int off = (min(kChunkSteps * c + kk, ks1 - ks0 - 1) - kk) * 16;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) r[j] = *(const u32x4*)(src[j] + off);
  };
  auto store = [&](const u32x4 (&r)[kPieces], int buf) {
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int p = tid + 256 * j, row = p / kParts, part = p % kParts;
      *(lds_u32x4*)(lds + buf * kStageB + row * kRowB + 16 * part) = r[j];
    }
  };
  f32x16 acc = f32x16{};
  auto compute = [&](int buf, int c) {
    const lds_u8* base = lds + buf * kStageB;
#pragma unroll
    for (int j = 0; j < kChunkSteps; ++j) {
      if (kChunkSteps * c + j < ks1 - ks0) {
        const bf16x8 a = *(const lds_bf16x8*)(base + (32 * ft + (lane & 31)) * kRowB + 32 * j + 16 * half);
        const bf16x8 b = *(const lds_bf16x8*)(base + (kGemmFeat + 32 * tt + (lane & 31)) * kRowB + 32 * j + 16 * half);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
    }
  };

  u32x4 ra[kPieces], rb[kPieces];
  if (n_chunks > 0) load(ra, 0);
  if (n_chunks > 1) load(rb, 1);
  if (n_chunks > 0) store(ra, 0);
  __syncthreads();
  for (int c = 0; c < n_chunks; c += 2) {
    // chunk c in buffer 0 (ra free), chunk c + 1 in flight in rb
    if (c + 2 < n_chunks) load(ra, c + 2);
    compute(0, c);
    if (c + 1 < n_chunks) store(rb, 1);
    __syncthreads();
    if (c + 1 >= n_chunks) break;
    // chunk c + 1 in buffer 1 (rb free), chunk c + 2 in flight in ra
    if (c + 3 < n_chunks) load(rb, c + 3);
    compute(1, c + 1);
    if (c + 2 < n_chunks) store(ra, 0);
    __syncthreads();
  }

  // lane holds token t0 + 32 tt + lane % 32, features f0 + 32 ft + 8 g + 4 half + 0..3
  const int t = t0 + 32 * tt + (lane & 31);
  if (t < n_tok) {
    if (go.part) {
      float* dst = go.part + ((int64_t)z * n_tok + t) * N + f0 + 32 * ft + 4 * half;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (f0 + 32 * ft + 8 * g + 4 * half + 4 <= N)
          *(f32x4*)(dst + 8 * g) = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    } else {
      const int dq = go.d_nope + go.d_rope, H = N / dq;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = f0 + 32 * ft + 8 * g + 4 * half;
        if (n + 4 > N) continue;
        const int s = n / dq, r = n % dq;
        u32x2 o;
        o[0] = (uint32_t)f32_to_bf16_bits(acc[4 * g]) | ((uint32_t)f32_to_bf16_bits(acc[4 * g + 1]) << 16);
        o[1] = (uint32_t)f32_to_bf16_bits(acc[4 * g + 2]) | ((uint32_t)f32_to_bf16_bits(acc[4 * g + 3]) << 16);
        uint16_t* dst = r < go.d_nope ? go.q_nope + ((int64_t)t * H + s) * go.d_nope + r
                                      : go.q_rope + ((int64_t)t * H + s) * go.d_rope + (r - go.d_nope);
        *(u32x2*)dst = o;
      }
    }
  }
}

// Epilogues: grid (ceil(N / 1024), n_tok), block 256; thread i of a work-group
// takes features 4i .. 4i+3 of the block's 1024 (the segment boundaries below
// are multiples of 4): the sum of the S partials in split order, rounded to bf16.
__device__ __forceinline__ bool sum_partials4(const float* __restrict__ part, int S, int n_tok, int N, int t, int n,
                                              u32x2* out) {
  if (n >= N) return false;
  // four splits' loads in flight at a time, summed in split order
  const float* p0 = part + (int64_t)t * N + n;
  const int64_t zs = (int64_t)n_tok * N;
  f32x4 v = *(const f32x4*)p0;
  int z = 1;
  for (; z + 3 < S; z += 4) {
    const f32x4 a = *(const f32x4*)(p0 + z * zs), b = *(const f32x4*)(p0 + (z + 1) * zs);
    const f32x4 c = *(const f32x4*)(p0 + (z + 2) * zs), d = *(const f32x4*)(p0 + (z + 3) * zs);
    v += a;
    v += b;
    v += c;
    v += d;
  }
  for (; z < S; ++z) v += *(const f32x4*)(p0 + z * zs);
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

// Split count: about 256 work-groups (one per CU; 512 and 1024 measured
// slower at 64 tokens: more, shorter work-groups and more partials) whatever
// the token count, at least two LDS stages per split.  A function of the
// shape only, so that the workspace size does not depend on the device.
int gemm_splits(int64_t n_tok, int64_t N, int64_t K) {
  const int64_t tiles = ((N + kGemmFeat - 1) / kGemmFeat) * ((n_tok + kGemmTok - 1) / kGemmTok);
  const int64_t ksteps = K / 16;
  int64_t s = (256 + tiles - 1) / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(1, ksteps / 16));   // at least two LDS stages per split
  return (int)std::max<int64_t>(s, 1);
}

void launch_gemm(const uint16_t* X, const uint16_t* W, int n_tok, int N, int K, int S, GemmOut go, hipStream_t st) {
  const int ksteps = K / 16;
  const int steps_per_split = (ksteps + S - 1) / S;
  dim3 grid((N + kGemmFeat - 1) / kGemmFeat, (n_tok + kGemmTok - 1) / kGemmTok, S);
  hipLaunchKernelGGL(xwt_gemm_kernel, grid, dim3(256), 0, st, X, W, n_tok, N, K, steps_per_split, go);
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
  GemmOut go{};
  go.part = part;
  launch_gemm(static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_down), n_tok, N, d_model, S, go, st);
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
  // (a single split writes the query parts directly: no partials)
  return (S > 1 ? up256((size_t)S * n_tok * N * 4) : 0) + up256((size_t)n_tok * d.n_heads * d.d_nope * 2) +
         up256((size_t)n_tok * d.n_heads * d.d_rope * 2);
}

mla_status launch_absorb_from_latent(const mla_dims& d, int32_t n_tok, int32_t d_cq, const void* c_q,
                                     const void* w_uq, const int32_t* pos, const void* w_uk, void* q_abs, void* ws,
                                     hipStream_t st) {
  const int N = d.n_heads * (d.d_nope + d.d_rope);
  const int S = gemm_splits(n_tok, N, d_cq);
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* part = reinterpret_cast<float*>(p);
  if (S > 1) p += up256((size_t)S * n_tok * N * 4);
  uint16_t* qn = reinterpret_cast<uint16_t*>(p);
  p += up256((size_t)n_tok * d.n_heads * d.d_nope * 2);
  uint16_t* qr = reinterpret_cast<uint16_t*>(p);
  GemmOut go{};
  if (S > 1) {
    go.part = part;
    launch_gemm(static_cast<const uint16_t*>(c_q), static_cast<const uint16_t*>(w_uq), n_tok, N, d_cq, S, go, st);
    hipLaunchKernelGGL(q_split_kernel, dim3((N + 1023) / 1024, n_tok), dim3(256), 0, st, part, S, n_tok, d.n_heads,
                       d.d_nope, d.d_rope, qn, qr);
  } else {   // one split: the GEMM writes the bf16 query parts itself
    go.q_nope = qn;
    go.q_rope = qr;
    go.d_nope = d.d_nope;
    go.d_rope = d.d_rope;
    launch_gemm(static_cast<const uint16_t*>(c_q), static_cast<const uint16_t*>(w_uq), n_tok, N, d_cq, S, go, st);
  }
  const mla_status s = launch_status();
  if (s != MLA_OK) return s;
  if (absorb_tuned_applies(d) && ((uintptr_t)w_uk & 15) == 0 && ((uintptr_t)q_abs & 15) == 0)
    return launch_absorb_tuned(d, n_tok, qn, qr, pos, w_uk, q_abs, st);
  return launch_absorb_generic(d, n_tok, qn, qr, pos, w_uk, q_abs, st);
}

}  // namespace mla
