// Prefill in the MHA form ("Transformer升级之路：21、MLA好在哪里？（下）",
// 双重投影, training/prefill column): every head attends with its own key
// [k_C | k_R], k_C = W_UK[s] c (d_nope = 128) and k_R the shared rotated key
// (d_R = 64), and its own value v = W_UV[s] c (d_v = 128); the query is
// [q_nope | RoPE(q_R)].  Queries and keys are packed per sequence (cu_q,
// cu_k): with Lq queries and Lk keys, query j sits at position Lk - Lq + j and
// attends to keys 0..Lk - Lq + j.  A whole prompt has Lq = Lk (query i at
// position i); a chunk of a longer prompt attends to the cached prefix too.
// The keys come either from packed c_KV / raw k_R rows (mla_prefill) or from
// the paged latent cache (mla_prefill_paged), whose k_R rows are already
// rotated.
//
// Launches:
// Precision: the latent and the weights enter the decompression as the bf16
// values they are; everything the attention contracts -- the query, k_C, the
// rotated k_R, v and the softmax weights -- is an fp16 operand of the matrix
// units (fp32 sums).  bf16 inputs convert to fp16 exactly (same exponent
// range for these magnitudes, 3 more significand bits), and each rounding of
// a computed operand (k_C, v, the weights, the rotated q_R) is 8 times finer
// than a bf16 one would be.  Computed operands must stay inside fp16's range
// (|x| < 65504).
//  1. prefill_rope_kernel: cos/sin of every query's RoPE pairs [Tq][32] (fp64
//     angle, fp32 cos/sin: the rule of the absorb and append kernels) and, for
//     packed keys, k_R' [Tk, 64] (fp64 rotation, rounded to fp32 and then to
//     bf16 as a bf16 cache stores it; kept as its exact fp16 value).  The
//     query's RoPE part is rotated by the attention kernel as it loads the
//     query (the pair formed in fp64, rounded to fp32, then to the fp16
//     operand).  For paged keys, prefill_gather_kernel packs each key's cache
//     row (latent and rotated k_R, the latter as fp16) into the workspace; an
//     fp8 latent is packed as its codes (exact in bf16) with the token's scale
//     beside it.
//  2. prefill_decompress_kernel: k_C [T, H, 128] and v [T, H, 128] in fp16, a
//     bf16 MFMA GEMM with fp32 accumulation: each wave holds its 32 weight rows
//     in registers, and the latent streams through LDS, 32 tokens at a time,
//     shared by the K and V waves of a head.  With an fp8 cache the fp32 sums
//     over the codes are multiplied by the token's scale before the rounding
//     (W (code * scale) = scale * (W code)).
//  3. prefill_attn_kernel: causal flash attention per (sequence, head, block of
//     128 queries), one wave per 32 queries; a work-group takes two query
//     blocks of its sequence, j and nq - 1 - j, so that every work-group has
//     the same causal work:
//     * key blocks of 64 rows [k_C | k_R | v] (640 B) are staged in LDS with
//       direct-to-LDS loads, two stages, in 1 KB blocks of 8 rows x 8 chunks
//       with the chunk XOR-swizzled by the row (the decode kernel's layout);
//       the next block's ten loads per wave go out one by one between the QK
//       MFMAs of the current one;
//     * S^T = K Q^T on MFMA 32x32x16 (queries in registers as the B operand);
//       the A operand reads key rows in the order that makes S^T come out in
//       the B-operand layout of PV (row R holds key R with bits 2 and 3
//       swapped), so the weights never leave the wave;
//     * online softmax in the exp2 domain with a lazy reference: the output is
//       rescaled only when a query's running max rises by more than 2^8;
//     * O^T += V^T P^T on MFMA, V^T from the staged rows by transpose reads;
//     * with an output gate (gated MLA), out = sigmoid(gate) * o before the
//       one rounding to bf16.
#include <algorithm>

#include "decode_tile.h"

namespace mla {
namespace {

constexpr int kPfDc = 512, kPfDn = 128, kPfDr = 64, kPfDv = 128;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f16x8 lds_f16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// fp16 bits of a float (round to nearest even)
__device__ __forceinline__ uint32_t f16_bits(float x) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x); }
// eight bf16 values (16 bytes) as eight fp16 values: exact for every bf16 inside fp16's normal range
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = f16_bits(__uint_as_float(v[i] << 16)) | (f16_bits(__uint_as_float(v[i] & 0xffff0000u)) << 16);
  return r;
}

// ---------------------------------------------------------------- 1. RoPE

// the sequence holding packed token t: the last b with cu[b] <= t
__device__ __forceinline__ int pf_seq_of(const int32_t* __restrict__ cu, int n_seq, int t) {
  int lo = 0, hi = n_seq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid;
  }
  return lo;
}

// One thread per (query token t, RoPE pair p): cos/sin of the pair's angle at
// the query's position go to cs[t][p] (float2), by the RoPE rule of the absorb
// and append kernels (fp64 angle, fp32 cos/sin); the attention kernel rotates
// the query's RoPE part with them as it loads the query.  k_rope non-null
// (packed keys, cu_k == cu_q, so the key of token t sits at the same
// position): the key pair is rotated here too (fp64 rotation, one rounding).
__global__ void __launch_bounds__(256) prefill_rope_kernel(const uint16_t* __restrict__ k_rope,
                                                           const int32_t* __restrict__ cu_q,
                                                           const int32_t* __restrict__ cu_k, int n_seq, int total_q,
                                                           float* __restrict__ cs, uint16_t* __restrict__ kr_out,
                                                           RopeFreqs f) {
  constexpr int kPairs = kPfDr / 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int t = (int)(i / kPairs), p = (int)(i % kPairs);
  if (t >= total_q) return;
  const int b = pf_seq_of(cu_q, n_seq, t);
  const int pos = (t - cu_q[b]) + (cu_k[b + 1] - cu_k[b]) - (cu_q[b + 1] - cu_q[b]);
  float c, sn;
  rope_cos_sin(pos, f.inv_freq[p], &c, &sn);
  *(float2*)(cs + 2 * i) = make_float2(c, sn);
  if (k_rope) {
    const int64_t at = (int64_t)t * kPfDr + 2 * p;
    const uint32_t x2 = *(const uint32_t*)(k_rope + at);
    float ox, oy;
    rope_pair(bf16_bits_to_f32((uint16_t)(x2 & 0xffffu)), bf16_bits_to_f32((uint16_t)(x2 >> 16)), c, sn, &ox, &oy);
    // rounded to bf16 as a bf16 cache stores it, then held as that value in fp16 (exact)
    *(uint32_t*)(kr_out + at) = f16_bits(bf16_bits_to_f32(f32_to_bf16_bits(ox))) |
                                (f16_bits(bf16_bits_to_f32(f32_to_bf16_bits(oy))) << 16);
  }
}

// Paged keys: one thread per (key token, 16-byte piece of its cache row):
// the row of key t (block_table[b][p / block_size] * block_size + p %
// block_size, p its position) is copied into the packed latent [t][d_c] and
// the packed rotated key [t][d_R] (the cache holds k_R already rotated).
// fp8 cache: the latent goes in as its E4M3FN codes, each exactly a bf16
// (16 codes per thread), and the token's scale to sc_out[t]; the
// decompression applies the scale to its fp32 sums.  A block-table entry
// outside [0, n_pool_blocks) is never read: its tokens get a zero latent and
// key (and scale 0).
template <bool kFp8>
__global__ void __launch_bounds__(256) prefill_gather_kernel(const uint8_t* __restrict__ pool, int64_t block_bytes,
                                                             int64_t n_pool_blocks,
                                                             const int32_t* __restrict__ block_table, int max_blocks,
                                                             int block_size, const int32_t* __restrict__ cu_k,
                                                             int n_seq, int total_k, uint16_t* __restrict__ c_out,
                                                             uint16_t* __restrict__ kr_out, float* __restrict__ sc_out) {
  constexpr int kCPieces = kFp8 ? kPfDc / 16 : kPfDc / 8;   // latent pieces (16 codes or 8 bf16 each)
  constexpr int kPieces = kCPieces + kPfDr / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int t = (int)(i / kPieces), piece = (int)(i % kPieces);
  if (t >= total_k) return;
  const int b = pf_seq_of(cu_k, n_seq, t);
  const int p = t - cu_k[b];
  const int64_t blk = block_table[(int64_t)b * max_blocks + p / block_size];
  const int slot = p % block_size;
  if (blk < 0 || blk >= n_pool_blocks) {   // padding inside the length (a caller error): zeros, nothing is read
    if (piece < kCPieces) {
      u32x4* dst = (u32x4*)(c_out + (int64_t)t * kPfDc + (kFp8 ? 16 : 8) * piece);
      dst[0] = u32x4{0, 0, 0, 0};
      if (kFp8) dst[1] = u32x4{0, 0, 0, 0};
      if (kFp8 && piece == 0) sc_out[t] = 0.f;
    } else {
      *(u32x4*)(kr_out + (int64_t)t * kPfDr + 8 * (piece - kCPieces)) = u32x4{0, 0, 0, 0};
    }
    return;
  }
  const uint8_t* base = pool + blk * block_bytes;
  if constexpr (!kFp8) {
    const u32x4 v = *(const u32x4*)(base + ((int64_t)slot * (kPfDc + kPfDr) + 8 * piece) * 2);
    if (piece < kCPieces) *(u32x4*)(c_out + (int64_t)t * kPfDc + 8 * piece) = v;
    else *(u32x4*)(kr_out + (int64_t)t * kPfDr + 8 * (piece - kCPieces)) = bf16x8_to_f16x8(v);
  } else {
    if (piece < kCPieces) {
      const u32x4 codes = *(const u32x4*)(base + (int64_t)slot * kPfDc + 16 * piece);
      if (piece == 0) sc_out[t] = *(const float*)(base + (int64_t)block_size * kPfDc + 4 * slot);
      uint32_t outw[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // scale 1: every E4M3FN code is exactly a bf16
        const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[w], 1.0f, false);   // codes 4w, 4w+1
        const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[w], 1.0f, true);    // codes 4w+2, 4w+3
        outw[2 * w] = *(const uint32_t*)&lo;
        outw[2 * w + 1] = *(const uint32_t*)&hi;
      }
      u32x4* dst = (u32x4*)(c_out + (int64_t)t * kPfDc + 16 * piece);
      dst[0] = u32x4{outw[0], outw[1], outw[2], outw[3]};
      dst[1] = u32x4{outw[4], outw[5], outw[6], outw[7]};
    } else {
      const int q = piece - kCPieces;
      *(u32x4*)(kr_out + (int64_t)t * kPfDr + 8 * q) = bf16x8_to_f16x8(
          *(const u32x4*)(base + (int64_t)block_size * (kPfDc + 4) + ((int64_t)slot * kPfDr + 8 * q) * 2));
    }
  }
}

// one direct-to-LDS load of 16 bytes per lane: LDS m0 + 16 lane <- src + voff
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t voff, uint32_t m0) {
  const uint64_t a = (uint64_t)(uintptr_t)src;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t sv = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane(m0);
  asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v], %[s]"
               :
               : [v] "v"(voff), [s] "s"(sv), [m] "s"(m)
               : "memory", "m0");
}
// the same load with no memory clobber, so that it can sit between the LDS reads
// and MFMAs of a block: the stage it writes is read by no one before the next
// barrier, which is itself ordered after it (both are volatile asm)
__device__ __forceinline__ void dma16_free(uint64_t sv, uint32_t voff, uint32_t m) {
  asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v], %[s]"
               :
               : [v] "v"(voff), [s] "s"(sv), [m] "s"(m)
               : "m0");
}
#pragma clang diagnostic pop

// a wave-uniform address in scalar registers
__device__ __forceinline__ uint64_t sgpr_addr(const void* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

// ---------------------------------------------------------------- 2. decompression

constexpr int kDcTok = 32;                   // tokens per LDS stage
constexpr int kDcStages = 4;                 // stage ring depth (three stages in flight)
constexpr int kDcStageB = kDcTok * kPfDc * 2;   // 32 KB: 32 latent rows of 1 KB
constexpr int kDcKs = kPfDc / 16;            // 32 k-steps
constexpr int kDcAhead = 8;                  // latent fragments read ahead of the MFMA chain

__device__ __forceinline__ u32x2 pf_pack4(float a, float b, float c, float d) {
  u32x2 r;
  r[0] = (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
  r[1] = (uint32_t)f32_to_bf16_bits(c) | ((uint32_t)f32_to_bf16_bits(d) << 16);
  return r;
}
__device__ __forceinline__ u32x2 pf_pack4_f16(float a, float b, float c, float d) {
  u32x2 r;
  r[0] = f16_bits(a) | (f16_bits(b) << 16);
  r[1] = f16_bits(c) | (f16_bits(d) << 16);
  return r;
}

// grid H * G, block 512 (8 waves).  Work-group (head s, token group g) writes
// k_C = W_UK[s] c (waves 0-3, dims 32 w ..) and v = W_UV[s] c (waves 4-7) for
// the 32-token tiles of group g.  Each wave keeps its 32 weight rows (the whole
// 512-long contraction, 128 VGPRs) in registers for the life of the
// work-group, so only the latent streams: 32 tokens x 1 KB per stage through a
// four-stage LDS ring filled by direct-to-LDS loads (one 1 KB row per
// instruction, 16-byte chunk p of row r holding logical chunk p ^ (r % 16), so
// that the 16 rows one 16-lane group reads at one chunk hit 16 different
// 16-byte slots of the LDS's 64 banks), three stages in flight.  The K and V halves share every latent tile; the work-groups of
// one token group run on one XCD and share the tiles in its L2.
__global__ void __launch_bounds__(512, 1) prefill_decompress_kernel(const uint16_t* __restrict__ c_kv,
                                                                    const float* __restrict__ tok_scale,
                                                                    const uint16_t* __restrict__ w_uk,
                                                                    const uint16_t* __restrict__ w_uv,
                                                                    uint16_t* __restrict__ kc, uint16_t* __restrict__ vv,
                                                                    int T, int H, int G) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[kDcStages * kDcStageB];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)lds_raw;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, lr = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u = xcd_unit(blockIdx.x, H * G);
  const int g = u / H, s = u % H;
  const int n_tiles = (T + kDcTok - 1) / kDcTok;
  const int j0 = (int)((int64_t)g * n_tiles / G), nt = (int)((int64_t)(g + 1) * n_tiles / G) - j0;
  if (nt <= 0) return;
  const bool is_v = wave >= 4;
  const int d0 = 32 * (wave & 3);

  // this wave's weight rows as MFMA A fragments: row d0 + lane % 32, k-step ks: elements 16 ks + 8 half .. +7
  bf16x8 af[kDcKs];
  {
    const bf16x8* wr = (const bf16x8*)((is_v ? w_uv : w_uk) + ((int64_t)s * kPfDv + d0 + lr) * kPfDc) + half;
#pragma unroll
    for (int ks = 0; ks < kDcKs; ++ks) af[ks] = wr[2 * ks];
  }
  __builtin_amdgcn_s_waitcnt(0);             // weights resident before the first stage load is queued

  // stage loads: wave w brings rows 4w .. 4w+3 of a tile, one row per instruction
  auto issue = [&](int j) {
    const uint32_t stage = lds0 + (uint32_t)((j % kDcStages) * kDcStageB);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * wave + rr;
      const int t = min((j0 + j) * kDcTok + r, T - 1);   // past the end: the last token (finite, not stored)
      dma16(c_kv + (int64_t)t * kPfDc, (uint32_t)(16 * (lane ^ (r & 15))), stage + (uint32_t)(r * 1024));
    }
  };
  // operations this wave queued after tile j's loads, when it waits for them: the
  // loads of tiles j+1, j+2 and the stores of tiles j-3 .. j-1 (four each)
  auto wait_tile = [&](int j) {
    const int n = min(2, nt - 1 - j) + min(3, j);
    switch (n) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<4>(); break;
      case 2: wait_vmcnt<8>(); break;
      case 3: wait_vmcnt<12>(); break;
      case 4: wait_vmcnt<16>(); break;
      default: wait_vmcnt<20>(); break;
    }
  };

  for (int j = 0; j < min(kDcStages - 1, nt); ++j) issue(j);
  uint16_t* out = (is_v ? vv : kc) + (int64_t)s * kPfDv + d0 + 4 * half;
  for (int j = 0; j < nt; ++j) {
    wait_tile(j);
    lds_barrier();                           // every wave's rows of tile j have landed; stage j-1 is free
    if (j + kDcStages - 1 < nt) issue(j + kDcStages - 1);
    const uint32_t stage = lds0 + (uint32_t)((j % kDcStages) * kDcStageB);
    const uint32_t brow = stage + (uint32_t)(lr * 1024);
    f32x16 acc = f32x16{};
    bf16x8 bf[kDcAhead];
#pragma unroll
    for (int ks = 0; ks < kDcAhead; ++ks)
      bf[ks] = *(const lds_bf16x8*)(uintptr_t)(brow + 16 * ((2 * ks + half) ^ (lr & 15)));
#pragma unroll
    for (int ks = 0; ks < kDcKs; ++ks) {
      const bf16x8 cur = bf[ks % kDcAhead];
      if (ks + kDcAhead < kDcKs)
        bf[ks % kDcAhead] = *(const lds_bf16x8*)(uintptr_t)(brow + 16 * ((2 * (ks + kDcAhead) + half) ^ (lr & 15)));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], cur, acc, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kDcAhead, 0);
#pragma unroll
    for (int ks = 0; ks < kDcKs - kDcAhead; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kDcAhead, 0);
    // lane holds token (j0 + j) 32 + lane % 32, dims d0 + 8 g + 4 half + 0..3 (g = i / 4); four
    // stores per tile (the clamped tokens of a partial last tile store to their own row: rows past
    // T are skipped by the lane's predicate, the instructions still issue)
    const int t = (j0 + j) * kDcTok + lr;
    if (t < T) {
      if (tok_scale) {                       // fp8 latent: the sums were over the codes
        const float sc = tok_scale[t];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] *= sc;
      }
      uint16_t* dst = out + (int64_t)t * H * kPfDv;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        *(u32x2*)(dst + 8 * gg) = pf_pack4_f16(acc[4 * gg], acc[4 * gg + 1], acc[4 * gg + 2], acc[4 * gg + 3]);
    }
  }
}

// ---------------------------------------------------------------- 3. attention

constexpr int kQBlk = 128;                   // queries per work-group (32 per wave)
constexpr int kKBlk = 64;                    // keys per stage
constexpr int kRowBlocks = 5;                // 1 KB blocks per 8 staged rows: k_C (2) | k_R (1) | v (2)
constexpr int kStage = kKBlk / 8 * kRowBlocks * 1024;   // 40960
constexpr int kQk = (kPfDn + kPfDr) / 16;    // 12 QK k-steps
constexpr int kKf = 8;                       // K fragments in flight ahead of the MFMA chain

// staged row r, 16-byte chunk c (c < 16: k_C, 16..23: k_R, 24..39: v); the
// row position and slot swizzle of the decode tile (rpos, swz), so 16 lanes
// reading 16 rows at one chunk hit 16 different slots
__device__ __forceinline__ uint32_t stage_off(int r, int c) {
  return ((r >> 3) * kRowBlocks + (c >> 3)) * 1024 + rpos(r) * 128 + 16 * ((c & 7) ^ swz(r & 7));
}

struct PrefillArgs {
  const uint16_t* q_nope;     // [T][H][128]
  const uint16_t* q_rope;     // [Tq][H][64] unrotated
  const float* cs;            // [Tq][32] (cos, sin) of each query's RoPE pairs
  const uint16_t* k_c;        // [T][H][128] fp16
  const uint16_t* k_rot;      // [T][64] rotated, fp16
  const uint16_t* v;          // [T][H][128] fp16
  const int32_t* cu_q;        // [n_seq + 1] query offsets
  const int32_t* cu_k;        // [n_seq + 1] key offsets
  const uint16_t* gate;       // [Tq][H][128] output-gate logits, or null
  uint16_t* out;              // [Tq][H][128]
  float* lse;                 // [Tq][H]
  int n_seq, H, n_qblk;       // n_qblk = ceil(max query length / 128)
  float scale_log2;
};



__global__ void __launch_bounds__(256, 2) prefill_attn_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[2 * kStage];
  lds_u8* lds = (lds_u8*)lds_raw;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, lr = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H;

  // work order: work-group j of a (sequence, head) takes its query blocks
  // nq - 1 - j and then j (nq = the sequence's own block count), so that under
  // the causal mask every work-group of a sequence has the same number of key
  // blocks and no long block is left alone at the end of the launch; all the
  // work-groups of one (sequence, head) run on one XCD, so the head's keys stay
  // in its L2
  const int n_slot = (a.n_qblk + 1) / 2;
  const int k = xcd_unit(blockIdx.x, a.n_seq * H * n_slot);
  const int pair = k / n_slot, j = k % n_slot;
  const int b = pair / H, s = pair % H;
  const int cu0 = a.cu_q[b], Lq = a.cu_q[b + 1] - cu0;
  const int ck0 = a.cu_k[b], L = a.cu_k[b + 1] - ck0;  // L keys; query i sits at position off + i
  const int off = L - Lq;
  const int nq = (Lq + kQBlk - 1) / kQBlk;
  if (j >= (nq + 1) / 2) return;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int qb = pass == 0 ? nq - 1 - j : j;
    if (pass == 1) {
      if (qb == nq - 1 - j) break;             // the middle block of an odd count: taken once
      lds_barrier();                           // every wave is done with the stages of the first block
    }
    const int q0 = qb * kQBlk;
    const int qw = q0 + 32 * wave;                       // this wave's first query
    const int q = min(qw + lr, Lq - 1);                  // this lane's query (past the end: a copy of the last)

    // queries: B operand, query q, dims 16k + 8 half .. +7 (k < 8: q_nope, else the rotated part)
    f16x8 qf[kQk];
    {
      const bf16x8* qn = (const bf16x8*)(a.q_nope + ((int64_t)(cu0 + q) * H + s) * kPfDn) + half;
      // the RoPE part, rotated here: k-step kk holds pairs 8 (kk - 8) + 4 half .. +3
      const bf16x8* qr = (const bf16x8*)(a.q_rope + ((int64_t)(cu0 + q) * H + s) * kPfDr) + half;
      const f32x4* csq = (const f32x4*)(a.cs + (int64_t)(cu0 + q) * kPfDr) + 2 * half;   // 2 pairs per f32x4
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 raw = qn[2 * kk];
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[kk][e] = (_Float16)(float)raw[e];   // exact
      }
#pragma unroll
      for (int kk = 8; kk < kQk; ++kk) {
        const bf16x8 raw = qr[2 * (kk - 8)];
        const f32x4 c01 = csq[4 * (kk - 8)], c23 = csq[4 * (kk - 8) + 1];
        const float cv[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
        f16x8 rot;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // the RoPE rule of the absorb: the pair formed in fp64, rounded to fp32, then to the fp16 operand
          float ox, oy;
          rope_pair((float)raw[2 * e], (float)raw[2 * e + 1], cv[2 * e], cv[2 * e + 1], &ox, &oy);
          // opaque: the compiler would otherwise fuse the two roundings into one float64 -> fp16
          // conversion, in software
          asm("" : "+v"(ox), "+v"(oy));
          rot[2 * e] = (_Float16)ox;
          rot[2 * e + 1] = (_Float16)oy;
        }
        qf[kk] = rot;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);             // queries resident before any stage load is queued

    // per-lane LDS offsets.  K (A operand of QK): row R = lr of a 32-key half reads
    // key R with bits 2 and 3 swapped; k-step kk reads chunk 2 kk + half.
    const int kr_row = (lr & ~12) | ((lr & 4) << 1) | ((lr & 8) >> 1);
    uint32_t kb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) kb[m] = stage_off(kr_row, 2 * m + half);
    // V^T (A operand of PV), dims 32 db + lane % 32, keys 16 ks + 8 half .. +7, as
    // two transpose reads (4 keys each); base by (db & 1, hh), + (db >> 1) KB, + 10 KB ks
    uint32_t vb[4];
    {
      const int gi = lane >> 4, sp = lane & 15;
      const int rr0 = 8 * (gi >> 1) + (sp >> 2);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int vdim = 32 * x + 16 * (gi & 1) + 4 * (sp & 3);
          vb[x * 2 + hh] = stage_off(rr0 + 4 * hh, 24 + (vdim >> 3)) + ((vdim & 7) << 1);
        }
    }

    // stage loads: wave w brings rows 16w .. 16w+15 of the block, five 1 KB
    // blocks per 8 rows; lane l (row position l/8): row 16w + 8g + ((l/8) ^ g),
    // logical chunk 8cb + ((l % 8) ^ swz(row % 8))
    const int last_key = min(L, off + q0 + kQBlk) - 1;
    const int n_kblk = last_key / kKBlk + 1;
    // A block's loads are prepared once (stage_prep: scalar sources, per-lane
    // offsets) and issued one at a time (stage_issue) between the QK MFMAs of the
    // block before, so that no wave stalls on ten load issues in a row.
    struct StageLd {
      uint64_t kc, kr, vv;          // k_C, k_R and v of the block's first key (wave-uniform)
      uint32_t off[2], roff[2], m0; // per-lane offsets of the k_C / v rows and the k_R row; LDS base
    };
    auto stage_prep = [&](int kbk, int par) -> StageLd {
      StageLd S;
      const int key0 = kbk * kKBlk;
      const int64_t row0 = ck0 + key0;
      S.kc = sgpr_addr(a.k_c + row0 * H * kPfDn);
      S.kr = sgpr_addr(a.k_rot + row0 * kPfDr);
      S.vv = sgpr_addr(a.v + row0 * H * kPfDv);
      S.m0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds + par * kStage) +
                                                      (uint32_t)(2 * wave * kRowBlocks * 1024));
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int rho = (lane >> 3) ^ g;           // the row (of 8) at position lane / 8 (rpos of row 8(2w + g) + rho)
        const int r = 16 * wave + 8 * g + rho;
        const int re = key0 + r < L ? r : 0;       // past the end: the block's first key (finite, masked)
        const int sl = (lane & 7) ^ swz(rho);
        // k_C chunks 0..15 and v chunks 24..39 (per-head rows of 256 B), k_R chunks 16..23 (128 B rows)
        S.off[g] = (uint32_t)((re * H + s) * (kPfDn * 2)) + 16 * sl;
        S.roff[g] = (uint32_t)(re * (kPfDr * 2)) + 16 * sl;
      }
      return S;
    };
    // load i = 5 g + j (a constant after unrolling): 1 KB block j of row group g
    auto stage_issue = [&](const StageLd& S, int i) {
      const int g = i / 5, j = i % 5;
      const uint32_t m = S.m0 + (uint32_t)((g * kRowBlocks + j) * 1024);
      if (j == 0) dma16_free(S.kc, S.off[g], m);
      else if (j == 1) dma16_free(S.kc, S.off[g] + 128, m);
      else if (j == 2) dma16_free(S.kr, S.roff[g], m);
      else if (j == 3) dma16_free(S.vv, S.off[g], m);
      else dma16_free(S.vv, S.off[g] + 128, m);
    };

    const float sl2 = a.scale_log2;
    float m_ref = -INFINITY, l_part = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x16{};

    // one key block; par = kbk % 2 is a constant in each of the two calls below, so the stage
    // base folds into the LDS instructions' immediate offsets
    auto block = [&](int kbk, int par) {
      wait_vmcnt<0>();                         // this wave's share of stage kbk has landed
      lds_barrier();                           // ... and everyone's; stage kbk-1 is free
      // the last block loads itself again into the free stage (never read), so that
      // the ten loads below need no branch
      const StageLd ld = stage_prep(min(kbk + 1, n_kblk - 1), par ^ 1);
      const uint32_t tb = (uint32_t)(uintptr_t)(lds + par * kStage);

      // ---- S^T for the two 32-key halves: one stream of 24 MFMAs with kKf K reads
      // in flight, the next block's ten loads after every other MFMA
      f32x16 sacc[2];
      auto kaddr = [&](int f) {
        const int t = f / kQk, kk = f % kQk;
        return tb + kb[kk % 4] + 1024 * (kk / 4) + 20480 * t;
      };
      f16x8 kf[kKf];
#pragma unroll
      for (int f = 0; f < kKf; ++f) kf[f] = *(const lds_f16x8*)(uintptr_t)kaddr(f);
#pragma unroll
      for (int f = 0; f < 2 * kQk; ++f) {
        const f16x8 cur = kf[f % kKf];
        if (f + kKf < 2 * kQk) kf[f % kKf] = *(const lds_f16x8*)(uintptr_t)kaddr(f + kKf);
        const int t = f / kQk, kk = f % kQk;
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur, qf[kk], kk == 0 ? f32x16{} : sacc[t], 0, 0, 0);
        if ((f & 1) && f / 2 < 10) stage_issue(ld, f / 2);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- softmax: lane holds query q, keys 64 kbk + 32 t + 16 (i / 8) + 8 half + i % 8
      float sv[2][16];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[t][i] = sacc[t][i];
      if (kbk * kKBlk + kKBlk - 1 > off + qw) {   // a block reaching this wave's diagonal (wave-uniform)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kbk * kKBlk + 32 * t + 16 * (i / 8) + 8 * half + (i % 8);
            sv[t][i] = key <= off + q ? sv[t][i] : -INFINITY;
          }
      }
      float bmax = sv[0][0];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) bmax = fmaxf(bmax, sv[t][i]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
        bmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float tmax = bmax * sl2;
      const bool raise = tmax > m_ref + 8.0f;  // also when nothing is accumulated yet (m_ref = -inf)
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? tmax : m_ref;
        const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= alpha;
        l_part *= alpha;
        m_ref = m_new;
      }
      const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
      f16x8 pb[4];                             // B operand of PV k-step 2t + j: regs 8j .. 8j+7 of half t
      const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          f16x8 v8;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const f32x2 pv = {__builtin_amdgcn_exp2f(fmaf(sv[t][8 * j + e], sl2, neg_m)),
                              __builtin_amdgcn_exp2f(fmaf(sv[t][8 * j + e + 1], sl2, neg_m))};
            const f16x2 p2 = __builtin_convertvector(pv, f16x2);   // round to nearest even; weights <= 2^8
            psum = __builtin_amdgcn_fdot2(p2, ones, psum, false);   // sum of the rounded weights
            v8[e] = p2[0];
            v8[e + 1] = p2[1];
          }
          pb[2 * t + j] = v8;
        }
      l_part += psum;

      // ---- O^T += V^T P^T: 4 dim blocks x 4 key steps
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint32_t base = tb + 10240 * ks + 1024 * (db >> 1);
          const f16x4 lo = __builtin_bit_cast(
              f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(base + vb[(db & 1) * 2])));
          const f16x4 hi = __builtin_bit_cast(
              f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(base + vb[(db & 1) * 2 + 1])));
          const f16x8 vf = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pb[ks], o[db], 0, 0, 0);
        }
    };
    {
      const StageLd ld0 = stage_prep(0, 0);
#pragma unroll
      for (int i = 0; i < 10; ++i) stage_issue(ld0, i);
    }
    for (int kbk = 0; kbk < n_kblk; kbk += 2) {
      block(kbk, 0);
      if (kbk + 1 < n_kblk) block(kbk + 1, 1);
    }

    wait_vmcnt<0>();                           // the last block's extra loads have landed
    // ---- normalise and store: O^T tile db, lane holds query qw + lr, dims 32 db + 8 (i / 4) + 4 half + i % 4
    float l_tot;
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
      l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (qw + lr < Lq) {
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      const int64_t at = ((int64_t)(cu0 + qw + lr) * H + s) * kPfDv + 4 * half;
      uint16_t* dst = a.out + at;
      if (a.gate) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const u32x2 g4 = *(const u32x2*)(a.gate + at + 32 * db + 8 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t w2 = g4[e >> 1];
              o[db][4 * g + e] *= sigmoid_f32(__uint_as_float((e & 1) ? (w2 & 0xffff0000u) : (w2 << 16)));
            }
          }
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(u32x2*)(dst + 32 * db + 8 * g) =
              pf_pack4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      if (half == 0)
        a.lse[(int64_t)(cu0 + qw + lr) * H + s] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    }
  }
}

}  // namespace

bool prefill_supported(const mla_dims& d) {
  return d.act_dtype == MLA_BF16 && d.d_c == kPfDc && d.d_nope == kPfDn && d.d_rope == kPfDr && d.d_v == kPfDv;
}

namespace {
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace: k_C, v [Tk][H][128] (fp16), the queries' (cos, sin) [Tq][32] (float2), k_R' [Tk][64] (fp16), then,
// for paged keys, the packed latent rows [Tk][d_c] (bf16) and the tokens' fp8 scales [Tk] (fp32); 256-byte
// aligned pieces
struct PrefillWs {
  uint16_t *kc, *vv, *kr;
  float* cs;
  uint16_t* ckv;   // paged keys: the packed latent rows
  float* sc;       // paged keys: the per-token scales of an fp8 latent
};
size_t prefill_ws_bytes(int64_t tq, int64_t tk, int64_t H, bool paged) {
  return up256(tk * H * kPfDn * 2) + up256(tk * H * kPfDv * 2) + up256(tq * kPfDr * 4) + up256(tk * kPfDr * 2) +
         (paged ? up256(tk * kPfDc * 2) + up256(tk * 4) : 0);
}
PrefillWs carve(void* ws, int64_t tq, int64_t tk, int64_t H) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  PrefillWs w;
  w.kc = reinterpret_cast<uint16_t*>(p);
  p += up256(tk * H * kPfDn * 2);
  w.vv = reinterpret_cast<uint16_t*>(p);
  p += up256(tk * H * kPfDv * 2);
  w.cs = reinterpret_cast<float*>(p);
  p += up256(tq * kPfDr * 4);
  w.kr = reinterpret_cast<uint16_t*>(p);
  p += up256(tk * kPfDr * 2);
  w.ckv = reinterpret_cast<uint16_t*>(p);
  p += up256(tk * kPfDc * 2);
  w.sc = reinterpret_cast<float*>(p);   // (carved past the end for packed keys, never used there)
  return w;
}

void launch_decompress(const mla_dims& d, const uint16_t* c_kv, const float* tok_scale, const void* w_uk,
                       const void* w_uv, const PrefillWs& w, int32_t total_k, hipStream_t st) {
  // token groups: about one work-group per CU (256) over the heads
  const int G = std::max(1, std::min(256 / std::max(d.n_heads, 1), (total_k + kDcTok - 1) / kDcTok));
  hipLaunchKernelGGL(prefill_decompress_kernel, dim3(d.n_heads * G), dim3(512), 0, st, c_kv, tok_scale,
                     static_cast<const uint16_t*>(w_uk), static_cast<const uint16_t*>(w_uv), w.kc, w.vv, total_k,
                     d.n_heads, G);
}

void launch_attention(const mla_dims& d, int32_t n_seq, const int32_t* cu_q, const int32_t* cu_k, int32_t max_q,
                      const void* q_nope, const void* q_rope, const PrefillWs& w, const void* gate, void* out,
                      float* lse, hipStream_t st) {
  PrefillArgs a;
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_rope = static_cast<const uint16_t*>(q_rope);
  a.cs = w.cs;
  a.k_c = w.kc;
  a.k_rot = w.kr;
  a.v = w.vv;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.gate = static_cast<const uint16_t*>(gate);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.n_seq = n_seq;
  a.H = d.n_heads;
  a.n_qblk = (max_q + kQBlk - 1) / kQBlk;
  a.scale_log2 = d.softmax_scale * 1.4426950408889634f;
  const int64_t grid = (int64_t)n_seq * d.n_heads * ((a.n_qblk + 1) / 2);
  hipLaunchKernelGGL(prefill_attn_kernel, dim3((unsigned)grid), dim3(256), 0, st, a);
}
}  // namespace

size_t prefill_workspace_bytes(const mla_dims& d, int64_t total_tokens) {
  return prefill_ws_bytes(total_tokens, total_tokens, d.n_heads, false);
}

size_t prefill_paged_workspace_bytes(const mla_dims& d, int64_t total_q, int64_t total_k) {
  return prefill_ws_bytes(total_q, total_k, d.n_heads, true);
}

mla_status launch_prefill(const mla_dims& d, int32_t n_seq, const int32_t* cu_seqlens, int32_t total_tokens,
                          int32_t max_seqlen, const void* q_nope, const void* q_rope, const void* c_kv,
                          const void* k_rope, const void* w_uk, const void* w_uv, const void* gate, void* ws,
                          void* out, float* lse, hipStream_t st) {
  const PrefillWs w = carve(ws, total_tokens, total_tokens, d.n_heads);
  const RopeFreqs f = make_rope_freqs(d);
  hipLaunchKernelGGL(prefill_rope_kernel, dim3((unsigned)(((int64_t)total_tokens * (kPfDr / 2) + 255) / 256)), dim3(256),
                     0, st, static_cast<const uint16_t*>(k_rope), cu_seqlens, cu_seqlens, n_seq, total_tokens, w.cs,
                     w.kr, f);
  launch_decompress(d, static_cast<const uint16_t*>(c_kv), nullptr, w_uk, w_uv, w, total_tokens, st);
  launch_attention(d, n_seq, cu_seqlens, cu_seqlens, max_seqlen, q_nope, q_rope, w, gate, out, lse, st);
  return launch_status();
}

mla_status launch_prefill_paged(const mla_dims& d, int32_t n_seq, const int32_t* cu_q, int32_t total_q, int32_t max_q,
                                const int32_t* cu_k, int32_t total_k, const void* q_nope, const void* q_rope,
                                const void* cache_pool, int64_t n_pool_blocks, const int32_t* block_table,
                                int32_t max_blocks,
                                const void* w_uk, const void* w_uv, const void* gate, void* ws, void* out, float* lse,
                                hipStream_t st) {
  const PrefillWs w = carve(ws, total_q, total_k, d.n_heads);
  const RopeFreqs f = make_rope_freqs(d);
  hipLaunchKernelGGL(prefill_rope_kernel, dim3((unsigned)(((int64_t)total_q * (kPfDr / 2) + 255) / 256)), dim3(256), 0,
                     st, nullptr, cu_q, cu_k, n_seq, total_q, w.cs, nullptr, f);
  const int64_t bb = (int64_t)mla_cache_block_bytes(&d);
  const uint8_t* pool8 = static_cast<const uint8_t*>(cache_pool);
  const bool f8 = d.cache_dtype == MLA_FP8_E4M3;
  if (f8)
    hipLaunchKernelGGL(prefill_gather_kernel<true>, dim3((unsigned)(((int64_t)total_k * 40 + 255) / 256)), dim3(256), 0,
                       st, pool8, bb, n_pool_blocks, block_table, max_blocks, d.block_size, cu_k, n_seq, total_k,
                       w.ckv, w.kr, w.sc);
  else
    hipLaunchKernelGGL(prefill_gather_kernel<false>, dim3((unsigned)(((int64_t)total_k * 72 + 255) / 256)), dim3(256), 0,
                       st, pool8, bb, n_pool_blocks, block_table, max_blocks, d.block_size, cu_k, n_seq, total_k,
                       w.ckv, w.kr, w.sc);
  launch_decompress(d, w.ckv, f8 ? w.sc : nullptr, w_uk, w_uv, w, total_k, st);
  launch_attention(d, n_seq, cu_q, cu_k, max_q, q_nope, q_rope, w, gate, out, lse, st);
  return launch_status();
}

}  // namespace mla
