// The log-sum-exp merge of the tuned decode kernel's split partials fused with
// the up-projection ("Transformer升级之路：21、MLA好在哪里？（下）", 双重投影,
// decoding column: o_t = W_UV o_lat per head after the latent attention), for
// d_c = 512, d_v = 128, bf16:
//   o_lat[t,s] = merge of the raw partials: M = max_k m_k, L = sum_k 2^(m_k - M) l_k,
//                o = sum_k 2^(m_k - M) O_k / L, rounded to bf16; lse = (M + log2 L) ln 2,
//   out[t,s,:] = W_UV[s] o_lat[t,s]  (times sigmoid(gate) with an output gate),
// in one launch.  Every element is computed with the operations, in the order,
// of combine_stream_kernel followed by up_proj_tuned_kernel, so the results
// are bit-identical to the two calls.
//
// One work-group of 8 waves per (head s, 32 query rows t of that head), one
// per CU.  Wave w merges rows 4w .. 4w+3 of the block: it brings the pieces of
// its rows straight into LDS (one 1 KB direct-to-LDS load per piece; four
// pieces per row per round, more rounds only for a row split over more than
// four work units), folds them in order against a running maximum (lane i
// owns latent dims 8i .. 8i+7), and leaves the merged bf16 row in the slot of
// its first piece.  A row the decode kernel finished itself (its sequence lies
// inside one work unit, or has no keys) is brought from o_lat instead.  The
// 1 KB row of block row j is stored with its 16-byte chunk c at position
// c ^ j, so the MFMA operand reads (16 rows at one chunk) hit 16 different
// LDS slots.  Waves 4-7 load their W_UV operands first, while the pieces are
// in flight, and after the merge multiply as the up-projection kernel does: wave 4 + w
// contracts latent dims 128w .. 128w+127 for the four output-row blocks, the
// four fp32 partial tiles are summed through LDS in a fixed order, and wave
// 4 + w finishes output rows 32w .. 32w+31.
#include <math.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) float lds_f32;

constexpr int kDc = 512, kDv = 128;
constexpr int kTok = 32;             // query rows (of one head) per work-group
constexpr int kRowsPerWave = 4;      // rows merged by each of the 8 waves
constexpr int kPieces = 4;           // pieces per row staged per round
constexpr int kSlotB = 1024;         // one latent row of bf16

struct CombineUpArgs {
  const uint16_t* ws_o;      // raw bf16 partials [slots][rows_per_seq][512]
  const float* ws_stats;     // [slots][rows_per_seq][2] = (m in log2 units, l)
  const int32_t* seqlens;
  const uint16_t* o_lat;     // [n_tok][H][512]: rows the decode kernel finished itself
  uint16_t* o_lat_out;       // merged rows written back here, or null
  const uint16_t* w_uv;      // [H][128][512]
  const uint16_t* gate;      // [n_tok][H][128] logits, or null
  uint16_t* out;             // [n_tok][H][128]
  float* lse;                // [n_tok][H]
  int n_seq, q_per_seq, H, n_tok;
  SplitLayout lay;
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

// one direct-to-LDS load of 16 bytes per lane: LDS m0 + 16 lane <- src + voff.
// Its completion is waited for with vmcnt; the slots it writes are read only by
// this wave, after that wait.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_row(const void* src, uint32_t voff, uint32_t m0) {
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
#pragma clang diagnostic pop

template <bool kGate>
__global__ void __launch_bounds__(512, 1) combine_up_proj_kernel(CombineUpArgs a) {
  // [32 rows][4 pieces][1 KB]; after the merge the MFMA waves' partial tiles reuse it
  __shared__ __attribute__((aligned(1024))) uint8_t stage_raw[kTok * kPieces * kSlotB];
  lds_u8* stage = (lds_u8*)stage_raw;
  const uint32_t stage0 = (uint32_t)(uintptr_t)stage;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int s = blockIdx.x, t0 = blockIdx.y * kTok;
  const int rows_per_seq = a.q_per_seq * a.H;

  constexpr int kVb = kDv / 32;                 // 4 output-row blocks
  constexpr int kSlice = kDc / 4;               // latent dims per MFMA wave
  constexpr int kSteps = kSlice / 16;           // 8 k-steps
  const bool mfma_wave = wave >= 4;
  const int mw = wave & 3;

  // ---- MFMA waves: this lane's W_UV operands, as the up-projection kernel loads them
  bf16x8 af[kVb][kSteps];
  if (mfma_wave) {
#pragma unroll
    for (int vb = 0; vb < kVb; ++vb) {
      const bf16x8* asrc =
          (const bf16x8*)(a.w_uv + ((int64_t)s * kDv + 32 * vb + (lane & 31)) * kDc + kSlice * mw) + half;
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) af[vb][ks] = asrc[2 * ks];
    }
  }
  {
    // ---- the merge of block rows 4w .. 4w+3 (row j: token t0 + j of sequence
    // t / q_per_seq).  The per-row and per-piece bookkeeping runs across lanes
    // (lane k < 4: row k; lane 4k + p < 16: piece p of row k in a round) and is
    // broadcast with readlane, so each lane does a few 64-bit divisions, not
    // one per piece.
    const int kl = lane & (kRowsPerWave - 1);
    const int jl = kRowsPerWave * wave + kl;                 // the block row of lane k
    const int tl = t0 + jl;
    const int bl = min(tl, a.n_tok - 1) / a.q_per_seq;
    // tiles of all sequences and before each row's sequence, with the decode kernel's
    // clamped lengths: the lanes take the sequences 64 apart, then sum across the wave
    int b_of[kRowsPerWave], before_k[kRowsPerWave] = {}, all = 0;
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k)
      b_of[k] = min(t0 + kRowsPerWave * wave + k, a.n_tok - 1) / a.q_per_seq;
    for (int i = lane; i < a.n_seq; i += 64) {
      const int32_t L = min(max(a.seqlens[i], 0), a.lay.max_len);
      const int nt = (L + a.lay.tile - 1) / a.lay.tile;
      all += nt;
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) before_k[k] += i < b_of[k] ? nt : 0;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      all += __shfl_xor(all, off, 64);
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) before_k[k] += __shfl_xor(before_k[k], off, 64);
    }
    int before = before_k[0];
#pragma unroll
    for (int k = 1; k < kRowsPerWave; ++k) before = kl == k ? before_k[k] : before;
    const int64_t total = all;
    const int64_t G = a.lay.n_splits;
    const int32_t Lb = min(max(a.seqlens[bl], 0), a.lay.max_len);
    const int nb = (Lb + a.lay.tile - 1) / a.lay.tile;
    const int64_t wf_l = nb > 0 ? unit_of_tile(before, total, G) : 0;
    const int64_t wl_l = nb > 0 ? unit_of_tile(before + nb - 1, total, G) : 0;
    const bool merge_l = tl < a.n_tok && nb > 0 && wl_l != wf_l;
    const int count_l = merge_l ? (int)(wl_l - wf_l + 1) : 0;
    // per row (wave-uniform): merge its pieces (units wf .. wf + count - 1), or copy it
    int wf[kRowsPerWave], count[kRowsPerWave];
    bool valid[kRowsPerWave], merge[kRowsPerWave];
    int rounds = 1;
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      valid[k] = t0 + kRowsPerWave * wave + k < a.n_tok;
      wf[k] = __builtin_amdgcn_readlane((int)wf_l, k);
      count[k] = __builtin_amdgcn_readlane(count_l, k);
      merge[k] = count[k] > 0;
      rounds = max(rounds, (count[k] + kPieces - 1) / kPieces);
    }
    // lane 4k + p (< 32) describes piece p of row k in a round
    const int kp = (lane >> 2) & (kRowsPerWave - 1), pp = lane & (kPieces - 1);
    const int wf_p = __builtin_amdgcn_ds_bpermute(4 * kp, (int)wf_l);
    const int count_p = __builtin_amdgcn_ds_bpermute(4 * kp, count_l);
    const int t_p = t0 + kRowsPerWave * wave + kp;
    const int b_p = min(t_p, a.n_tok - 1) / a.q_per_seq;
    const int r_p = (t_p % a.q_per_seq) * a.H + s;

    float m[kRowsPerWave], tot[kRowsPerWave];
    f32x4 acc[kRowsPerWave][2];
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      m[k] = -INFINITY;
      tot[k] = 0.f;
      acc[k][0] = acc[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int rd = 0; rd < rounds; ++rd) {
      if (rd > 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's reads of its slots are done
      // this lane's piece of the round: its partial row, whether its unit owns a
      // tile (a unit that owns none left nothing in its slot), its statistics
      const int pc_p = kPieces * rd + pp;
      const bool in_p = lane < kPieces * kRowsPerWave && pc_p < count_p;
      const int64_t w_p = (int64_t)wf_p + pc_p;
      const int64_t row_p = (w_p + b_p) * rows_per_seq + r_p;
      const bool owns_p = in_p && unit_first_tile(w_p, total, G) < unit_first_tile(w_p + 1, total, G);
      f32x2 st_l = f32x2{0.f, 0.f};
      if (owns_p) st_l = *(const f32x2*)(a.ws_stats + row_p * 2);
      const uint64_t owners = __ballot(owns_p);
      // the pieces of this round into their slots (a row that is copied: its o_lat row, in round 0)
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) {
        const int j = kRowsPerWave * wave + k;    // block row
        const uint32_t voff = (uint32_t)(16 * (lane ^ j));
#pragma unroll
        for (int p = 0; p < kPieces; ++p) {
          const uint32_t m0 = stage0 + (uint32_t)((kPieces * j + p) * kSlotB);
          if ((owners >> (kPieces * k + p)) & 1) {
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)row_p, kPieces * k + p);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)row_p >> 32), kPieces * k + p);
            const int64_t row = (int64_t)(((uint64_t)hi << 32) | lo);
            dma_row(a.ws_o + row * kDc, voff, m0);
          } else if (p == 0 && rd == 0 && valid[k] && !merge[k]) {
            dma_row(a.o_lat + ((int64_t)(t0 + j) * a.H + s) * kDc, voff, m0);
          }
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // every piece (and the statistics) has landed
      // fold the round's pieces in order, as the merge kernel does
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) {
        const int j = kRowsPerWave * wave + k;
#pragma unroll
        for (int p = 0; p < kPieces; ++p) {
          if (!((owners >> (kPieces * k + p)) & 1)) continue;
          const float sm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(st_l[0]), kPieces * k + p));
          const float sl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(st_l[1]), kPieces * k + p));
          if (!(sl > 0.f)) continue;
          const u32x4 raw = *(const lds_u32x4*)(stage + (kPieces * j + p) * kSlotB + 16 * (lane ^ j));
          const float mn = fmaxf(m[k], sm);
          const float keep = exp2f(m[k] - mn);   // 0 while nothing is accumulated (m = -inf)
          const float wgt = exp2f(sm - mn);
          tot[k] = fmaf(tot[k], keep, wgt * sl);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t w2 = raw[e >> 1];
            const float x = (e & 1) ? bf_hi(w2) : bf_lo(w2);
            acc[k][e >> 2][e & 3] = fmaf(acc[k][e >> 2][e & 3], keep, wgt * x);
          }
          m[k] = mn;
        }
      }
    }
    // the merged rows (bf16) into their first slot, lse to memory
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      const int j = kRowsPerWave * wave + k;
      if (!merge[k]) continue;
      const float inv = tot[k] > 0.f ? 1.0f / tot[k] : 0.f;
      u32x4 o;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        o[2 * h] = pack2(acc[k][h][0] * inv, acc[k][h][1] * inv);
        o[2 * h + 1] = pack2(acc[k][h][2] * inv, acc[k][h][3] * inv);
      }
      *(lds_u32x4*)(stage + (kPieces * j) * kSlotB + 16 * (lane ^ j)) = o;
      const int t = t0 + j;
      if (a.o_lat_out) *((u32x4*)(a.o_lat_out + ((int64_t)t * a.H + s) * kDc) + lane) = o;
      if (lane == 0) a.lse[(int64_t)t * a.H + s] = tot[k] > 0.f ? (m[k] + log2f(tot[k])) * 0.69314718055994530942f : -INFINITY;
    }
  }
  __syncthreads();   // every merged row is in LDS

  // ---- the up-projection of the 32 merged rows
  bf16x8 bf[kSteps];
  if (mfma_wave) {
    // B operand: block row lane % 32, latent dims 128 mw + 16 ks + 8 half .. +7 (chunk 16 mw + 2 ks + half)
    const int j = lane & 31;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks)
      bf[ks] = *(const lds_bf16x8*)(stage + (kPieces * j) * kSlotB + 16 * ((16 * mw + 2 * ks + half) ^ j));
  }
  __syncthreads();   // the merged rows are read: the stage takes the partial tiles
  lds_f32* red = (lds_f32*)stage;               // [wave][vb][reg][lane], 64 KB
  if (mfma_wave) {
    f32x16 accm[kVb];
#pragma unroll
    for (int vb = 0; vb < kVb; ++vb) accm[vb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
      for (int vb = 0; vb < kVb; ++vb) accm[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[vb][ks], bf[ks], accm[vb], 0, 0, 0);
#pragma unroll
    for (int vb = 0; vb < kVb; ++vb)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[((mw * kVb + vb) * 16 + i) * 64 + lane] = accm[vb][i];
  }
  __syncthreads();   // the four MFMA waves' partial tiles are in LDS
  if (!mfma_wave) return;
  // output-row block vb = mw: rows 32 vb + 8 (i / 4) + 4 half + i % 4, token lane % 32
  const int t = t0 + (lane & 31);
  const int tc = min(t, a.n_tok - 1);
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = red[((0 * kVb + mw) * 16 + i) * 64 + lane];
#pragma unroll
    for (int w2 = 1; w2 < 4; ++w2) x += red[((w2 * kVb + mw) * 16 + i) * 64 + lane];
    v[i] = x;
  }
  if constexpr (kGate) {
    const uint16_t* gsrc = a.gate + ((int64_t)tc * a.H + s) * kDv + 32 * mw + 4 * half;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 graw = *(const u32x2*)(gsrc + 8 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w2 = graw[e >> 1];
        v[4 * g + e] *= sigmoid_f32((e & 1) ? bf_hi(w2) : bf_lo(w2));
      }
    }
  }
  if (t < a.n_tok) {
    uint16_t* dst = a.out + ((int64_t)t * a.H + s) * kDv + 32 * mw + 4 * half;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 r;
      r[0] = pack2(v[4 * g], v[4 * g + 1]);
      r[1] = pack2(v[4 * g + 2], v[4 * g + 3]);
      *(u32x2*)(dst + 8 * g) = r;
    }
  }
}

}  // namespace

bool combine_up_proj_applies(const mla_dims& d, const DecodePlan& plan) {
  return plan.kind == 1 && plan.layout.mode == 1 && d.act_dtype == MLA_BF16 && d.d_c == kDc && d.d_v == kDv;
}

mla_status launch_combine_up_proj(const mla_dims& d, const DecodePlan& plan, int32_t n_seq, int32_t q_per_seq,
                                  const int32_t* seqlens, const void* ws, const void* o_lat, void* o_lat_out,
                                  const void* w_uv, const void* gate, void* out, float* lse, hipStream_t st) {
  const int n_tok = n_seq * q_per_seq;
  CombineUpArgs a;
  a.ws_o = static_cast<const uint16_t*>(ws);
  a.ws_stats = static_cast<const float*>(ws) + plan.ws_stats_offset_floats;
  a.seqlens = seqlens;
  a.o_lat = static_cast<const uint16_t*>(o_lat);
  a.o_lat_out = static_cast<uint16_t*>(o_lat_out);
  a.w_uv = static_cast<const uint16_t*>(w_uv);
  a.gate = static_cast<const uint16_t*>(gate);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.n_seq = n_seq;
  a.q_per_seq = q_per_seq;
  a.H = d.n_heads;
  a.n_tok = n_tok;
  a.lay = plan.layout;
  dim3 grid(d.n_heads, (n_tok + kTok - 1) / kTok);
  if (gate)
    hipLaunchKernelGGL(combine_up_proj_kernel<true>, grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL(combine_up_proj_kernel<false>, grid, dim3(512), 0, st, a);
  return launch_status();
}

}  // namespace mla
