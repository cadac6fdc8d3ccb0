// Tuned gfx950 latent-attention decode for a 512-wide latent plus a 64-wide
// shared RoPE key in bf16 (the absorbed form of MLA: every head attends with
// key [c | k_R] (576 wide) and value c (512 wide), shared by all heads).
//
// Work decomposition (one work-group = 4 waves = one per SIMD of a CU):
//  * The key tiles (32 tokens) of all sequences are laid end to end and cut
//    into `units` equal runs (stream-K); a run may cover several sequences or
//    a piece of one.  A sequence lying inside one run gets its final output
//    written here; otherwise each piece writes (o, lse) partials for the
//    log-sum-exp combine.
//  * A work-group serves 128 (query row, head) "pairs": all 128 heads of one
//    query row, or 64 heads x 2 rows (grid.y picks the head group).
//  * HBM -> LDS: each tile (32 rows x 1152 B, contiguous inside a paged block)
//    is copied with 16-byte direct-to-LDS loads into a 4-stage ring.  In LDS a
//    tile is a grid of 1 KB blocks, each holding 8 rows x 8 sixteen-byte
//    chunks; rows r and r + 8 of a tile sit in different halves of their 1 KB
//    blocks and the chunk position is XOR-swizzled by the row, so the K reads
//    and the V transpose reads below hit distinct LDS banks within each group
//    of 16 lanes, and one wave loads a whole 1 KB block per instruction.
//  * S^T = K Q^T on bf16 MFMA 32x32x16: wave w owns pairs 32w..32w+31 and
//    keeps their queries in registers as the B operand; the K tile is the A
//    operand (one 16-byte LDS read per lane per k-step).  With all 128 pairs
//    in one work-group (bf16 cache) the score tile is kept in VGPRs (the MFMAs
//    are written as assembly), so that the 16 output tiles own the 256 AGPRs,
//    and the nine loads of tile T+2 are issued one at a time between the
//    MFMAs of QK(T) instead of in one burst after the barrier.
//  * Online softmax in the exp2 domain against a per-pair reference max fixed
//    by the first tile that shows the pair a key; P = 2^(z - ref) is rounded
//    to bf16 and exchanged through LDS.  Should a later tile exceed the
//    reference by more than 2^16, the reference is raised and the sequence
//    piece is computed once more (never in practice; it keeps the result
//    exact without ever rescaling the accumulators, which inside the tile
//    loop are only ever MFMA-updated or zeroed; they are read out once, in
//    the epilogue).
//  * O^T += V^T P^T on bf16 MFMA 32x32x16: wave w owns latent dims
//    128w..128w+127 for all 128 pairs (fp32 accumulators, 256 per lane); V^T
//    comes straight from the row-major tile with the LDS transpose read.
//  * fp8 cache (E4M3FN codes with one fp32 scale per token, bf16 k_R): a
//    token's score is scale * <q_lat, code> + <q_R, k_R> and its value is
//    scale * code, so the codes enter both contractions exactly as bf16 and the
//    scale multiplies the latent part of the score and the PV weight.  With 128
//    pairs per work-group the staged tile (codes, k_R, scales: 24 KB) is read in
//    place: one 16-byte code read per lane feeds the A operands of two QK
//    k-steps (the queries are loaded in the same dim order), converted to bf16
//    in registers, and each V^T fragment is one 8-bit LDS transpose read,
//    converted the same way.  With fewer pairs the tile is first expanded to
//    the bf16 layout in LDS.
#include <type_traits>

#include "decode_tile.h"

namespace mla {
namespace {

constexpr int kStages = 4;
constexpr int kPairs = 128;
constexpr int kPRow = 64;                                   // bytes per P row: 32 bf16, 16-byte chunks XOR-swizzled
constexpr int kPBufBytes = kPairs * kPRow;                  // 8192
constexpr int kQSteps = kDk / 16;                           // 36 k-steps of the QK contraction
constexpr int kKAhead = 8;                                  // K fragment reads in flight per wave
static_assert(kKAhead % 4 == 0, "K prefetch depth is a multiple of the 4 per-lane read bases");

constexpr int kOffP = kStages * kTileBytes;                 // 147456: two P buffers (tile T in buffer T % 2)
constexpr int kLdsBytes = kOffP + 2 * kPBufBytes;           // 163840
// fp8 cache, tiles expanded in LDS (fewer than 4 pair blocks): two bf16 tile
// buffers (tile T in buffer T % 2), then a 3-slot staging ring for the raw
// tiles, ending where the P buffers start
constexpr int kF8Slots = 3;
constexpr int kOffF = 2 * kTileBytes;
static_assert(kOffF + kF8Slots * kF8StageBytes == kOffP, "fp8 buffers use the bf16 ring's space");
// fp8 cache read in place (4 pair blocks): a ring of kStages raw stages
static_assert(kStages * kF8StageBytes <= kOffP, "fp8 stages fit below the P buffers");
// Small scratch shares P buffer 0; it is used only while no weights are live
// there: the sequence scan before the first tile, the redo flags after the
// last PV of an attempt, the (l, m) rows in the piece epilogue.
constexpr int kOffL = kOffP;                                // 128 floats
constexpr int kOffM = kOffL + kPairs * 4;                   // 128 floats
constexpr int kOffFlag = kOffM + kPairs * 4;                // 4 ints
constexpr int kOffScan = kOffFlag + 16;                     // 4 ints
constexpr int kOffMisc = kOffScan + 16;                     // 2 ints
static_assert(kOffMisc + 8 <= kOffP + kPBufBytes, "scratch inside P buffer 0");

// epilogue staging: one row of 512 bf16 per pair, padded by 16 bytes (bf16
// cache); 64 rows of 512 fp32, padded by 16 bytes so that 8 lanes writing 8
// consecutive rows at one column hit 8 different 16-byte slots (fp8 cache)
constexpr int kYRow = kDc * 2 + 16;
static_assert(kPairs * kYRow <= kOffP, "epilogue staging fits in the tile stages");
constexpr int kXRow = kDc * 4 + 16;
static_assert(64 * kXRow <= kOffP, "epilogue staging fits in the tile stages");

constexpr float kRestartThreshold = 16.0f;                  // log2 units: weights stay <= 2^16

static_assert(kTile == 32, "the MFMA tiling below assumes 32-token tiles");
static_assert(kLdsBytes <= 163840, "LDS budget of a gfx950 CU");

struct Args {
  const uint16_t* q_abs;        // [n_seq][q_per_seq][H][576] bf16
  const uint8_t* pool;          // paged cache, block_bytes per block
  uint16_t* o_final;            // [n_seq][q_per_seq][H][512] bf16
  float* lse_final;             // [n_seq][q_per_seq][H]
  uint16_t* ws_o;               // partials [slots][q_per_seq*H][512] bf16, raw (relative to 2^m)
  float* ws_stats;              // partials [slots][q_per_seq*H][2] = (m in log2 units, l)
  int64_t block_bytes;
  int64_t n_pool_blocks;        // block ids outside [0, n_pool_blocks) are padding, never read
  int32_t max_blocks, block_size, n_seq, q_per_seq, n_heads, units, heads_per_wg;
  float scale_log2;             // softmax_scale * log2(e)
};

// wait until at most n tiles' worth of this wave's loads are still in flight
__device__ __forceinline__ void wait_tiles(int n) {
  if (n >= 3) wait_vmcnt<3 * kLoadsPerWave>();
  else if (n == 2) wait_vmcnt<2 * kLoadsPerWave>();
  else if (n == 1) wait_vmcnt<kLoadsPerWave>();
  else wait_vmcnt<0>();
}


__device__ __forceinline__ void wait_tiles_fp8(int n) {
  if (n >= 3) wait_vmcnt<3 * kF8LoadsPerWave>();
  else if (n == 2) wait_vmcnt<2 * kF8LoadsPerWave>();
  else if (n == 1) wait_vmcnt<kF8LoadsPerWave>();
  else wait_vmcnt<0>();
}

// QK with the score tile in VGPRs, written as assembly so that the compiler
// cannot place the accumulator in AGPRs (those hold the 16 output tiles).
// Back-to-back MFMAs accumulating into the same registers need no wait states;
// the chain starts from the inline constant 0.  The vector ALU may read the
// result only after the last MFMA has written it: mfma_to_valu waits 24
// states, more than an 8-pass XDL op requires.  The A/B operands come from LDS
// reads and global loads, never from vector ALU writes.
__device__ __forceinline__ void mfma_qk_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// the same, for an A operand written by vector ALU instructions (two wait states first)
__device__ __forceinline__ void mfma_qk_first_n(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk_n(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_to_valu(f32x16& acc) { asm volatile("s_nop 15\n\ts_nop 7" : "+v"(acc)); }

template <bool kFp8, int kPB>
__global__ void __launch_bounds__(256, 1) decode576_kernel(Args a, const int32_t* __restrict__ block_table,
                                                          const int32_t* __restrict__ seqlens) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[kLdsBytes];
  // fp8 cache, 4 pair blocks: the codes are read in place and converted to
  // bf16 in registers (kF8D); the other fp8 instantiations expand each tile
  // to bf16 in LDS first (kF8X)
  constexpr bool kF8D = kFp8 && kPB == 4;
  constexpr bool kF8X = kFp8 && !kF8D;
  lds_u8* lds = (lds_u8*)lds_raw;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.units;
  // Work-groups are handed to the 8 XCDs round-robin by their linear index;
  // consecutive units (the pieces of one sequence, which read the same
  // queries) are given to work-groups of one XCD so they share its L2.
  const int unit = xcd_unit(blockIdx.x, G), hg = blockIdx.y;
  const int32_t max_len = a.max_blocks * a.block_size;
  // block ids are 32-bit: a pool of 2^31 blocks or more bounds nothing below INT32_MAX
  const int32_t npool32 = a.n_pool_blocks < INT32_MAX ? (int32_t)a.n_pool_blocks : INT32_MAX;
  // sequence length as used here: clamped to what the block table can address
  auto seq_len = [&](int b) -> int32_t { return min(max(seqlens[b], 0), max_len); };

  // ---- tiles per sequence: exclusive scan over sequences (chunked per thread)
  const int chunk = (a.n_seq + 255) / 256;
  const int s_lo = min(tid * chunk, a.n_seq), s_hi = min(s_lo + chunk, a.n_seq);
  int local = 0;
  for (int b = s_lo; b < s_hi; ++b) local += tiles_of(seq_len(b));
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  lds_i32* scan = (lds_i32*)(lds + kOffScan);
  if (lane == 63) scan[wave] = incl;
  lds_barrier();
  int wave_off = 0;
  for (int w = 0; w < wave; ++w) wave_off += scan[w];
  // Tile indices are 32-bit (the host bounds the tile count below 2^31); the
  // count and the unit's range are wave-uniform and live in scalar registers.
  const int N = __builtin_amdgcn_readfirstlane(scan[0]) + __builtin_amdgcn_readfirstlane(scan[1]) +
                __builtin_amdgcn_readfirstlane(scan[2]) + __builtin_amdgcn_readfirstlane(scan[3]);
  const int excl = wave_off + incl - local;
  const int T0 = (int)unit_first_tile(unit, N, G), T1 = (int)unit_first_tile(unit + 1, N, G);
  lds_i32* misc = (lds_i32*)(lds + kOffMisc);
  if (local > 0 && T0 >= excl && T0 < excl + local) {
    int start = excl, b = s_lo;
    while (start + tiles_of(seq_len(b)) <= T0) { start += tiles_of(seq_len(b)); ++b; }
    misc[0] = b;
    misc[1] = start;
  }
  lds_barrier();
  if (T0 >= T1) return;                    // an empty unit (more units than tiles)
  int b_first = __builtin_amdgcn_readfirstlane(misc[0]);
  int b_first_start = __builtin_amdgcn_readfirstlane(misc[1]);

  // ---- per-wave identity of its 32 QK pairs; each lane owns pair 32*wave + lane%32.
  // The work-group serves 32 * kPB pairs; waves 0 .. kPB-1 run QK and the
  // softmax for theirs, all four run PV.  With kPB < 4 a pair past the last
  // query row (heads x rows fewer than the pairs) is padding: it repeats the
  // last row's work and stores nothing.  kPB = 4 is only used without padding.
  const int hpw = a.heads_per_wg;
  const bool qk_wave = kPB == 4 || wave < kPB;
  const int my_pair = 32 * wave + (lane & 31);
  const int my_j_raw = my_pair / hpw;
  const bool pad = kPB == 4 ? false : my_j_raw >= a.q_per_seq;
  const int my_j = kPB == 4 ? my_j_raw : min(my_j_raw, a.q_per_seq - 1);
  const int my_s = hg * hpw + my_pair % hpw;
  const int half = lane >> 5;
  const int rows_per_seq = a.q_per_seq * a.n_heads;

  // per-lane LDS byte offsets (within a tile / the P buffer) of the operand reads
  uint32_t kq_base[4];                     // K rows: row lane%32, chunk 8*(k/4) + 2*(k%4) + half
  {
    const int r = lane & 31;
#pragma unroll
    for (int m = 0; m < 4; ++m) kq_base[m] = tile_off(r, 2 * m + half);
  }
  uint32_t v_base[4];                      // V^T transpose reads, by (db & 1, hh), for ks = 0, db < 2
  {
    const int gi = lane >> 4, sp = lane & 15;
    const int dim = 128 * wave + 16 * (gi & 1) + 4 * (sp & 3);   // + 32 db
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 8 * (gi >> 1) + 4 * hh + (sp >> 2);     // + 16 ks
        v_base[x * 2 + hh] = tile_off(row, (dim + 32 * x) >> 3) + ((dim & 7) << 1);
      }
  }
  // P buffer rows: pair r holds its 32 weights (bf16) as 4 chunks of 16 bytes,
  // logical chunk c stored at c ^ ((r >> 2) & 3), so 16 consecutive rows at one
  // chunk cover 16 distinct 16-byte slots.
  const int psw = ((lane & 31) >> 2) & 3;
  // writer: row my_pair, tokens 8qq + 4*half .. +3 of the tile (8 bytes at chunk qq)
  const uint32_t p_wr = (uint32_t)(uintptr_t)(lds + kOffP) + my_pair * kPRow + 8 * half;
  // reader (PV B operand): row 32pb + lane%32, tokens 16ks + 8*half .. +7, i.e.
  // chunk (2ks + half) ^ psw = 2 (ks ^ (psw >> 1)) + (half ^ (psw & 1)); the
  // per-ks offset 32 (ks ^ (psw >> 1)) is the ks = 0 base plus 32 ks, negated
  // when psw >> 1 is set
  const uint32_t p_rd = (uint32_t)(uintptr_t)(lds + kOffP) + (lane & 31) * kPRow + 16 * (half ^ (psw & 1)) +
                        32 * (psw >> 1);
  const int p_ks_sign = (psw >> 1) ? -1 : 1;
  // fp8 in place: K code reads (row lane % 32, chunk 2m + half; chunk pair j adds 1 KB per 4),
  // k_R reads (chunk 2m + half), V^T transpose reads (dim block db: 16 lanes bring 8 rows x 16 codes)
  uint32_t f8_cb[4], f8_rb[4], f8_vb[4];
  if constexpr (kF8D) {
    const int r = lane & 31;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f8_cb[m] = f8_code_off(r, 2 * m + half);
      f8_rb[m] = f8_rope_off(r, 2 * m + half);
    }
    const int g = lane >> 4, i = lane & 15;
    const int row = 8 * (g >> 1) + (i >> 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) f8_vb[db] = f8_code_off(row, 8 * wave + 2 * db + (g & 1)) + 8 * (i & 1);
  }

  const float sl2 = a.scale_log2;
  lds_f32* s_l = (lds_f32*)(lds + kOffL);
  lds_f32* s_m = (lds_f32*)(lds + kOffM);
  lds_i32* s_flag = (lds_i32*)(lds + kOffFlag);

  // O^T tiles [db][pb] for dims 128*wave + 32*db, pairs 32*pb.  With 16
  // tiles (kPB = 4) they fill the 256 AGPRs, so the score tile (and, for an
  // fp8 cache, the RoPE part of the scores) lives in VGPRs: the QK MFMAs are
  // written as assembly (kAsmQK).  The accumulators are only ever
  // MFMA-updated, zeroed, or stored raw.
  constexpr bool kAsmQK = kPB == 4;
  constexpr int kOAcc = 4 * kPB;
  f32x16 o[kOAcc];
  bf16x8 q[kQSteps];

  // ---- the pieces: one per sequence overlapping [T0, T1)
  int b = b_first;
  int seq_start = b_first_start;
  for (;;) {
    const int32_t L = seq_len(b);
    const int seq_end = seq_start + tiles_of(L);
    const int p0 = seq_start > T0 ? seq_start : T0;
    const int p1 = seq_end < T1 ? seq_end : T1;
    const bool whole = seq_start >= T0 && seq_end <= T1;
    const int32_t* bt_row = block_table + (int64_t)b * a.max_blocks;

    float m_ref = -INFINITY, l_part = 0.f;
    // a block-table entry names a block of the pool (else it is padding: its tokens are masked, never read)
    auto in_pool = [&](int32_t blk) { return blk >= 0 && (int64_t)blk < a.n_pool_blocks; };
    // rows of tile T that hold tokens of the sequence (0 for a padding block entry)
    auto tile_valid = [&](int T) -> int {
      const int tok0 = (int)(T - seq_start) * kTile;
      return in_pool(bt_row[tok0 / a.block_size]) ? min(kTile, L - tok0) : 0;
    };
    // bit T % kStages: tile T lies in a padding block (bf16 cache; the fp8
    // cache masks such rows through their scales)
    uint32_t stage_pad = 0;
    // fp8 in place: byte T % kStages holds tile T's valid row count
    uint32_t stage_valid = 0;
    // issue this wave's share of the loads of tile T: bf16 straight into ring
    // stage T % kStages; fp8 into staging slot T % 3 (expanded later)
    // Load cursor (bf16 cache): the block-table position of the next tile to
    // load, with the entry after it fetched one block ahead, so that issuing a
    // tile's loads never waits for a block-table read and needs no division.
    int c_pos = 0, c_sub = 0;
    int32_t c_blk = -1, c_nxt = -1;
    const int tpb = a.block_size / kTile;              // tiles per cache block
    auto cursor_at = [&](int T) {
      const int t = T - seq_start;
      c_pos = t / tpb;
      c_sub = t - c_pos * tpb;
      c_blk = bt_row[c_pos];
      c_nxt = c_pos + 1 < a.max_blocks ? bt_row[c_pos + 1] : -1;
    };
    if constexpr (!kF8X) cursor_at(p0);
    // bf16 (and fp8 in place): prepare the loads of tile T (the cursor's tile) and advance the cursor
    auto load_prep = [&](int T) {
      const int tok0 = (int)(T - seq_start) * kTile;
      const bool ok = c_blk >= 0 && c_blk < npool32;
      const int valid = ok ? min(kTile, L - tok0) : 0;
      const uint8_t* blkp = ok ? a.pool + (int64_t)c_blk * a.block_bytes : a.pool;
      const int slot = ok ? c_sub * kTile : 0;
      const uint32_t bit = 1u << (T % kStages);
      stage_pad = valid == 0 ? (stage_pad | bit) : (stage_pad & ~bit);
      const uint32_t sh = 8u * (uint32_t)(T % kStages);
      stage_valid = (stage_valid & ~(0xffu << sh)) | ((uint32_t)valid << sh);
      if (++c_sub == tpb) {
        c_sub = 0;
        ++c_pos;
        c_blk = c_nxt;
        c_nxt = c_pos + 1 < a.max_blocks ? bt_row[c_pos + 1] : -1;
      }
      if constexpr (kF8D) {
        return tile_f8_prep(blkp, slot, a.block_size, valid, lds + (int)(T % kStages) * kF8StageBytes, wave, lane);
      } else {
        return tile_part_prep(blkp + (int64_t)slot * kRowBytes, valid, lds + (int)(T % kStages) * kTileBytes, wave,
                              lane);
      }
    };
    using LoadT = decltype(load_prep(0));
    auto load_tile = [&](int T) {
      if constexpr (kF8D) {
        const TileF8 p = load_prep(T);
#pragma unroll
        for (int i = 0; i < kF8LoadsPerWave; ++i) tile_f8_issue(p, i);
      } else if constexpr (!kFp8) {
        const TilePart p = load_prep(T);
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) tile_part_issue(p, i);
      } else {
        const int tok0 = (int)(T - seq_start) * kTile;
        const int32_t blk = bt_row[tok0 / a.block_size];
        const bool ok = in_pool(blk);
        const uint8_t* bp = ok ? a.pool + (int64_t)blk * a.block_bytes : a.pool;
        issue_tile_fp8(bp, ok ? tok0 % a.block_size : 0, a.block_size, tile_valid(T),
                       lds + kOffF + (int)(T % kF8Slots) * kF8StageBytes, wave, lane);
      }
    };
    // wait until at most n tiles' loads of this wave are still in flight
    auto wait_tile = [&](int n) {
      if constexpr (!kFp8) wait_tiles(n);
      else wait_tiles_fp8(n);
    };
    // fp8: staged tile T -> bf16 buffer T % 2
    auto expand = [&](int T) {
      expand_tile_fp8(lds + kOffF + (int)(T % kF8Slots) * kF8StageBytes, lds + (int)(T & 1) * kTileBytes, wave);
    };
    // LDS address of tile T's bf16 image
    auto tile_base = [&](int T) -> uint32_t {
      if constexpr (kF8D) return (uint32_t)(uintptr_t)(lds + (int)(T % kStages) * kF8StageBytes);
      const int slot = kFp8 ? (int)(T & 1) : (int)(T % kStages);
      return (uint32_t)(uintptr_t)(lds + slot * kTileBytes);
    };

    // The first tiles of the piece are queued right behind the queries, so
    // the two fetches overlap; one full wait then leaves the compiler no query
    // load pending inside the tile loop.
    // queries of this sequence: B operand fragments, pair my_pair, dims 16k + 8*half .. +7
    if (qk_wave) {
      const int64_t row = ((int64_t)b * a.q_per_seq + my_j) * a.n_heads + my_s;
      const bf16x8* src = (const bf16x8*)(a.q_abs + row * kDk) + half;
#pragma unroll
      for (int k = 0; k < kQSteps; ++k) {
        // fp8 in place: latent k-step 2j + e takes dims 32j + 16 half + 8e .. +7 (one 16-byte code read
        // serves both k-steps of a pair); the query follows the same order
        if constexpr (kF8D) q[k] = k < 32 ? src[4 * (k >> 1) + half + (k & 1)] : src[2 * k];
        else q[k] = src[2 * k];
      }
    }
    int pre = 0;                         // tiles of the first attempt already issued
    for (; pre < kStages - 2 && p0 + pre < p1; ++pre) load_tile(p0 + pre);
    __builtin_amdgcn_s_waitcnt(0);           // queries and the first tiles resident

    for (;;) {                               // attempts: a second one only after a reference jump
#pragma unroll
      for (int i = 0; i < kOAcc; ++i) o[i] = f32x16{};
      l_part = 0.f;
      int T_issue = p0 + pre;            // loads in flight cover [T, T_issue)
      pre = 0;                               // a second attempt loads every tile again
      bool redo = false;                     // a reference jumped during this attempt (wave-uniform)

      // ---- softmax of tile T against the reference max (exp2 domain); the
      // weights go to P buffer T % 2.  The scale is positive (checked by the
      // API), so the max of the raw scores gives the max of the scaled ones and
      // the scale folds into one FMA per weight.
      auto softmax = [&](const f32x16& sacc, const float (&s_rope)[16], int T) {
        const int tok0 = (int)(T - seq_start) * kTile;
        float sv[16], sc[16];
        if constexpr (kFp8) {
          // this lane's 16 token scales (rows past the tile's valid ones hold
          // no data: scale 0 and score -inf)
          const lds_u8* scl = kF8D ? lds + (int)(T % kStages) * kF8StageBytes + kF8OffScales + 1024 * wave
                                   : lds + kOffF + (int)(T % kF8Slots) * kF8StageBytes + kF8OffScales + 1024 * wave;
          const int nv = kF8D ? (int)((stage_valid >> (8 * (T % kStages))) & 0xffu) : tile_valid(T);
          auto scale_scores = [&](auto full_c) {
            constexpr bool kFull = decltype(full_c)::value;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 s4 = *(const lds_f32x4*)(scl + 4 * (8 * g + 4 * half));
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bool in = kFull || 8 * g + 4 * half + e < nv;
                sc[4 * g + e] = in ? s4[e] : 0.f;
                sv[4 * g + e] = in ? fmaf(sacc[4 * g + e], s4[e], s_rope[4 * g + e]) : -INFINITY;
              }
            }
          };
          // a full tile (wave-uniform test) needs no per-row mask
          if (nv == kTile) scale_scores(std::true_type{});
          else scale_scores(std::false_type{});
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
          if ((stage_pad >> (T % kStages)) & 1u) {   // a tile of a padding block (wave-uniform): all masked
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[i] = -INFINITY;
          }
        }
        // causal / length mask: only a tile reaching past the first query row's
        // last visible token needs it (wave-uniform test)
        if (tok0 + kTile > L - a.q_per_seq + 1) {
          // the lane's row and token offsets are derived here from an opaque copy of the
          // lane id: kept across the tile loop (the compiler would carry the visible count
          // as a per-lane induction variable) they can be spilled, and the reload's
          // memory-count wait, placed inside the loop, waits for every tile load in flight
          int lx = lane;
          asm volatile("" : "+v"(lx));
          const int mj = kPB == 4 ? (32 * wave + (lx & 31)) / hpw : min((32 * wave + (lx & 31)) / hpw, a.q_per_seq - 1);
          const int vis = L - a.q_per_seq + mj - tok0 + 1;  // tokens [0, vis) of this tile are visible
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int t = 8 * (i / 4) + 4 * (lx >> 5) + (i % 4);
            sv[i] = t < vis ? sv[i] : -INFINITY;
          }
        }
        // the reference is set by the first tile that shows this pair a key; a
        // later jump by more than 2^16 raises it (weights stay <= 2^16) and
        // marks the piece for a second pass
        auto ref_update = [&]() {
          float smax = sv[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) smax = fmaxf(smax, sv[i]);
          // the pair's other 16 tokens live in lane l ^ 32
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
          smax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
          const float tmax = smax * sl2;
          const bool had_ref = m_ref != -INFINITY;
          const bool grow = tmax > m_ref + kRestartThreshold;
          if (grow) m_ref = tmax;
          redo |= __builtin_amdgcn_ballot_w64(grow && had_ref) != 0;
        };
        // bf16 cache, every pair of the wave with a reference: the weights are
        // taken against it right away, and the tile max only when a lane's
        // sum of rounded weights reaches 2^16 (a weight above 2^16 rounds to at
        // least 2^16, so no jump goes unseen); the rule applied is the same
        const bool fast = (!kFp8 || kF8D) && __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) == 0;
        if (!fast) ref_update();
        // exp2 of masked scores is 0; an unset reference (no visible key yet) is taken as 0
        const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
        float psum = 0.f;
        uint32_t pk[8];
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const f32x2 pv = {__builtin_amdgcn_exp2f(fmaf(sv[i], sl2, neg_m)),
                            __builtin_amdgcn_exp2f(fmaf(sv[i + 1], sl2, neg_m))};
          if constexpr (kFp8) {
            // the value is code x scale: the scale goes into the PV weight
            psum += pv[0] + pv[1];
            const bf16x2 pb2 = __builtin_convertvector(f32x2{pv[0] * sc[i], pv[1] * sc[i + 1]}, bf16x2);
            pk[i / 2] = *(const uint32_t*)&pb2;
          } else {
            const bf16x2 pb2 = __builtin_convertvector(pv, bf16x2);              // round to nearest even
            psum = __builtin_amdgcn_fdot2_f32_bf16(pb2, ones, psum, false);     // sum of the rounded weights
            pk[i / 2] = *(const uint32_t*)&pb2;
          }
        }
        if (fast && __builtin_amdgcn_ballot_w64(psum >= 65536.f) != 0) ref_update();
        l_part += psum;
        const uint32_t pw = p_wr + (uint32_t)(T & 1) * kPBufBytes;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const u32x2 v2 = {pk[2 * qq], pk[2 * qq + 1]};
          *(lds_u32x2*)(uintptr_t)(pw + 16 * (qq ^ psw)) = v2;
        }
      };

      // ---- O^T += V^T P^T for tile T: this wave's 128 dims x all 128 pairs
      auto pv = [&](uint32_t tb, int T) {
        if constexpr (kF8D) {
          // fp8 in place.  V^T fragment (k-step ks, dim block db): one 8-bit transpose read
          // (lane: dim 32 db + lane % 32 of this wave's 128, tokens 16 ks + 8 half .. +7),
          // converted to bf16.  The first k-step's P fragments and all eight transpose reads go
          // out first, the second k-step's P fragments once its MFMAs have started.
          const uint32_t pbuf = p_rd + (uint32_t)(T & 1) * kPBufBytes;
          bf16x8 pf0[kPB], pf1[kPB];
#pragma unroll
          for (int pb = 0; pb < kPB; ++pb) pf0[pb] = *(const lds_bf16x8*)(uintptr_t)(pbuf + 32 * pb * kPRow);
          i32x2_t v[2][4];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int db = 0; db < 4; ++db)
              v[ks][db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(uintptr_t)(tb + f8_vb[db] + 8192 * ks));
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int db = 0; db < 4; ++db) {
              const bf16x8 vf = f8x8_to_bf16((uint32_t)v[ks][db][0], (uint32_t)v[ks][db][1]);
#pragma unroll
              for (int pb = 0; pb < kPB; ++pb)
                o[db * kPB + pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, ks ? pf1[pb] : pf0[pb], o[db * kPB + pb],
                                                                           0, 0, 0);
              if (ks == 0 && db == 0) {
#pragma unroll
                for (int pb = 0; pb < kPB; ++pb)
                  pf1[pb] = *(const lds_bf16x8*)(uintptr_t)(pbuf + (uint32_t)(32 * p_ks_sign) + 32 * pb * kPRow);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          return;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 pf[kPB];
          const uint32_t pbuf = p_rd + (uint32_t)(T & 1) * kPBufBytes + (uint32_t)(32 * ks * p_ks_sign);
#pragma unroll
          for (int pb = 0; pb < kPB; ++pb) pf[pb] = *(const lds_bf16x8*)(uintptr_t)(pbuf + 32 * pb * kPRow);
          // V^T fragments for the 4 dim blocks: two transpose reads each (4 tokens apiece)
          bf16x4 h[8];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int x = 0; x < 4; ++x)
              h[hh * 4 + x] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                  (lds_bf16x4*)(uintptr_t)(tb + v_base[x] + 2 * 9 * 1024 * ks + 1024 * hh));
          // h[x*2 + hh] (+ 4 for dim blocks 2, 3): block db uses h[(db >> 1) * 4 + (db & 1) * 2 + hh]
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const bf16x4 lo = h[(db >> 1) * 4 + (db & 1) * 2], hi = h[(db >> 1) * 4 + (db & 1) * 2 + 1];
            const bf16x8 vf = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int pb = 0; pb < kPB; ++pb)
              o[db * kPB + pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[pb], o[db * kPB + pb], 0, 0, 0);
          }
        }
      };

      // tiles ahead of the first: two when the loop issues during QK (kAsmQK), else three
      while (T_issue - p0 < (kAsmQK ? kStages - 2 : kStages - 1) && T_issue < p1) load_tile(T_issue++);
      wait_tile(T_issue - 1 - p0);           // tile p0 has landed
      lds_barrier();
      if constexpr (kF8X) {
        expand(p0);
        lds_barrier();
      }

      // bf16: one barrier per tile, after the weights are written: it
      // publishes P(T) (buffer T % 2) and tile T+1 (each wave waits for its own
      // loads of it first), and every wave has finished PV(T-1) by then, so the
      // next tile load goes into the stage of T-1.
      // fp8: two barriers per tile.  The first (after the weights are written)
      // publishes P(T) and the staged tile T+1; the expansion of tile T happened
      // before the previous second barrier, so the next staging load goes into
      // the slot of T, and tile T+1 is expanded into the bf16 buffer of T-1
      // (whose PV also finished before it).  The second publishes the expanded
      // tile T+1 and ends PV(T).
      if constexpr (kAsmQK) {
        // bf16, 4 pair blocks: the loads of tile T+2 go out one by one between
        // the MFMAs of QK(T), into the stage of T-2 (free since the previous
        // barrier); one barrier per tile publishes P(T) and tile T+1.
        for (int T = p0; T < p1; ++T) {
          const uint32_t tb = tile_base(T);
          f32x16 sacc;
          float s_rope[16];
          auto qk = [&](const LoadT* lp) {
            if constexpr (kF8D) {
              // fp8 in place: the 4 RoPE k-steps (bf16 k_R) into their own sum, then the 32 latent
              // k-steps, each 16-byte code read converted into the A operands of a k-step pair; the
              // conversion of pair j+1 runs while the MFMAs of pair j do.  The tile's six loads go
              // out between them.
              f32x16 srope;
              bf16x8 kr[4];
#pragma unroll
              for (int m = 0; m < 4; ++m) kr[m] = *(const lds_bf16x8*)(uintptr_t)(tb + f8_rb[m]);
              u32x4 raw[2];
              raw[0] = *(const lds_u32x4*)(uintptr_t)(tb + f8_cb[0]);
              raw[1] = *(const lds_u32x4*)(uintptr_t)(tb + f8_cb[1]);
#pragma unroll
              for (int m = 0; m < 4; ++m) {
                if (m == 0) mfma_qk_first(srope, kr[0], q[32]);
                else mfma_qk(srope, kr[m], q[32 + m]);
                __builtin_amdgcn_sched_barrier(0);
              }
              bf16x8 a0 = f8x8_to_bf16(raw[0][0], raw[0][1]), a1 = f8x8_to_bf16(raw[0][2], raw[0][3]);
              raw[0] = *(const lds_u32x4*)(uintptr_t)(tb + f8_cb[2]);
#pragma unroll
              for (int j = 0; j < 16; ++j) {
                if (j == 0) mfma_qk_first_n(sacc, a0, q[0]);
                else mfma_qk_n(sacc, a0, q[2 * j]);
                mfma_qk_n(sacc, a1, q[2 * j + 1]);
                if (lp != nullptr && j % 3 == 0) tile_f8_issue(*lp, j / 3);
                if (j + 1 < 16) {
                  const u32x4 w = raw[(j + 1) & 1];
                  if (j + 3 < 16) raw[(j + 1) & 1] = *(const lds_u32x4*)(uintptr_t)(tb + f8_cb[(j + 3) & 3] + 1024 * ((j + 3) >> 2));
                  a0 = f8x8_to_bf16(w[0], w[1]);
                  a1 = f8x8_to_bf16(w[2], w[3]);
                }
                __builtin_amdgcn_sched_barrier(0);
              }
              mfma_to_valu(sacc);
#pragma unroll
              for (int i = 0; i < 16; ++i) s_rope[i] = srope[i];
              return;
            }
            bf16x8 kf[kKAhead];
#pragma unroll
            for (int k = 0; k < kKAhead; ++k) kf[k] = *(const lds_bf16x8*)(uintptr_t)(tb + kq_base[k % 4] + 1024 * (k / 4));
#pragma unroll
            for (int k = 0; k < kQSteps; ++k) {
              const bf16x8 cur = kf[k % kKAhead];
              if (k == 0) mfma_qk_first(sacc, cur, q[k]);
              else mfma_qk(sacc, cur, q[k]);
              if (k + kKAhead < kQSteps)
                kf[k % kKAhead] = *(const lds_bf16x8*)(uintptr_t)(tb + kq_base[k % 4] + 1024 * ((k + kKAhead) / 4));
              if constexpr (!kF8D) {
                if (lp != nullptr && k % 4 == 1) tile_part_issue(*lp, k / 4);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
            mfma_to_valu(sacc);
          };
          if (T_issue < p1) {
            const LoadT lp = load_prep(T_issue++);
            qk(&lp);
          } else {
            qk(nullptr);
          }
          softmax(sacc, s_rope, T);
          if (T + 1 < p1) wait_tile(T_issue - 2 - T);   // tile T+1 has landed (T+2 may be in flight)
          lds_barrier();
          pv(tb, T);
        }
      } else {
      for (int T = p0; T < p1; ++T) {
        const uint32_t tb = tile_base(T);
        if (qk_wave) {
          // ---- S^T = K Q^T for this wave's 32 pairs: lane holds pair my_pair, tokens 8(i/4)+4*half+i%4.
          // K-step k reads logical chunk 2k + half of row lane%32: chunk group k/4
          // adds 1 KB, so four per-lane bases (by k%4) plus immediates suffice.
          // fp8: the 4 RoPE k-steps (32..35) run first into their own sum, since
          // only the latent part of a key is scaled (z = s_t <q_lat, code> + <q_R, k_R>).
          f32x16 sacc = {};
          float s_rope[16];
          {
            // kKAhead K fragments in flight ahead of the MFMA chain (the LDS is
            // shared by the four waves, whose reads queue behind each other)
            bf16x8 kf[kKAhead];
#pragma unroll
            for (int k = 0; k < kKAhead; ++k) {
              const int kk = kFp8 ? (k + 32) % kQSteps : k;   // (kk % 4 == k % 4)
              kf[k] = *(const lds_bf16x8*)(uintptr_t)(tb + kq_base[k % 4] + 1024 * (kk / 4));
            }
#pragma unroll
            for (int k = 0; k < kQSteps; ++k) {
              const int kk = kFp8 ? (k + 32) % kQSteps : k;
              const int kn = kFp8 ? (k + kKAhead + 32) % kQSteps : k + kKAhead;
              const bf16x8 cur = kf[k % kKAhead];
              if (k + kKAhead < kQSteps)
                kf[k % kKAhead] = *(const lds_bf16x8*)(uintptr_t)(tb + kq_base[k % 4] + 1024 * (kn / 4));
              sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, q[kk], sacc, 0, 0, 0);
              if constexpr (kFp8) {
                if (k == 3) {
#pragma unroll
                  for (int i = 0; i < 16; ++i) s_rope[i] = sacc[i];
                  sacc = f32x16{};
                }
              }
            }
            // issue order: kKAhead reads, then (MFMA, read) pairs, then the last kKAhead MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, kKAhead, 0);
#pragma unroll
            for (int k = 0; k < kQSteps - kKAhead; ++k) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kKAhead, 0);
          }
          softmax(sacc, s_rope, T);
        }
        if (T + 1 < p1) wait_tile(T_issue - 2 - T);   // (staged) tile T+1 has landed (later ones may be in flight)
        lds_barrier();
        if (T_issue < p1) load_tile(T_issue++);
        if constexpr (kFp8) {
          if (T + 1 < p1) expand(T + 1);
        }
        pv(tb, T);
        if constexpr (kFp8) lds_barrier();
      }
      }
      wait_vmcnt<0>();
      lds_barrier();                         // every wave is done with the last tile and P (the flags share P buffer 0)
      if (lane == 0) s_flag[wave] = redo ? 1 : 0;
      lds_barrier();
      const bool any_redo = (s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3]) != 0;
      lds_barrier();                         // flags read
      if (!any_redo) break;
      if constexpr (!kF8X) cursor_at(p0);    // the second attempt loads from the first tile again
      // Some pair's reference rose by more than 2^16 after it had accumulated
      // weights: run the piece again.  Every reference now lies within 2^16 of
      // its pair's maximum over the piece, so the second pass cannot jump.
    }

    // The epilogue derives its lane-dependent values again from an opaque copy
    // of the lane id, so that the compiler does not compute them ahead of the
    // tile loop and hold them (spilled to scratch) across it.
    int lane_x = lane;
    asm volatile("" : "+v"(lane_x));
    const int e_half = lane_x >> 5;
    const int e_pair = 32 * wave + (lane_x & 31);
    const int e_j_raw = e_pair / hpw;
    const bool e_pad = kPB == 4 ? false : e_j_raw >= a.q_per_seq;
    const int e_j = kPB == 4 ? e_j_raw : min(e_j_raw, a.q_per_seq - 1);
    const int e_s = hg * hpw + e_pair % hpw;
    const int e_tid = 64 * wave + lane_x;
    // ---- finish the piece.  The accumulators go out through LDS (free now:
    // every load has landed and every wave is past the last tile): each lane
    // rounds its pair's values to bf16 into one 1 KB row per pair, so that each
    // store instruction writes 1 KB of one output row instead of 32-byte pieces
    // of 32 rows.  A piece that is a whole sequence is normalised on the way
    // (bf16 o_lat and lse); any other piece leaves its raw partial (relative to
    // 2^m) and (m, l) in slot unit + b.
    const int64_t slot_row0 = (int64_t)(unit + b) * rows_per_seq;
    float l_tot;
    {
      // the pair's other 16 tokens were summed in lane l ^ 32
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
      l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (lane_x < 32 && qk_wave) {
      if (!whole && !e_pad) {
        const int my_row = e_j * a.n_heads + e_s;
        a.ws_stats[(slot_row0 + my_row) * 2] = m_ref;
        a.ws_stats[(slot_row0 + my_row) * 2 + 1] = l_tot;
      }
      s_l[e_pair] = l_tot;
      s_m[e_pair] = m_ref;
    }
    if constexpr (!kF8X) {
      lds_barrier();                               // every pair's l is in LDS
      // a partial is stored raw (a factor of 1 is exact), a whole sequence normalised
      const bool norm = whole;
      auto stage = [&](auto norm_c) {
      constexpr bool kNorm = decltype(norm_c)::value;
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) {
        const int pair = 32 * pb + (lane_x & 31);
        const float inv = kNorm ? (s_l[pair] > 0.f ? 1.0f / s_l[pair] : 0.f) : 1.0f;
        // lane: dims 128 wave + 32 db + 8 (i / 4) + 4 half + i % 4 of its pair
        lds_u8* yrow = lds + pair * kYRow + (128 * wave + 4 * e_half) * 2;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            f32x4 v = f32x4{o[db * kPB + pb][4 * qq], o[db * kPB + pb][4 * qq + 1], o[db * kPB + pb][4 * qq + 2],
                            o[db * kPB + pb][4 * qq + 3]};
            // hardware pack, round to nearest even
            if constexpr (kNorm) v = v * inv;
            const bf16x2 lo = __builtin_convertvector(f32x2{v[0], v[1]}, bf16x2);
            const bf16x2 hi = __builtin_convertvector(f32x2{v[2], v[3]}, bf16x2);
            *(lds_u32x2*)(yrow + (32 * db + 8 * qq) * 2) = u32x2{*(const uint32_t*)&lo, *(const uint32_t*)&hi};
          }
      }
      };
      if (norm) stage(std::true_type{});
      else stage(std::false_type{});
      lds_barrier();                                // the rows (and s_l, s_m) are in LDS
      {
        // thread t: 16-byte chunk t % 64 of rows t / 64 + 4k (one wave writes one 1 KB row)
        const int c = e_tid & 63;
        uint16_t* const dst0 = (norm ? a.o_final + (int64_t)b * rows_per_seq * kDc : a.ws_o + slot_row0 * kDc) + 8 * c;
#pragma unroll 4
        for (int k = 0; k < 8 * kPB; ++k) {
          const int pair = (e_tid >> 6) + 4 * k;
          if (kPB != 4 && pair / hpw >= a.q_per_seq) continue;   // padding
          const int row_in_seq = (pair / hpw) * a.n_heads + hg * hpw + pair % hpw;
          const u32x4 v = *(const lds_u32x4*)(lds + pair * kYRow + c * 16);
          *(u32x4*)(dst0 + (int64_t)row_in_seq * kDc) = v;
        }
      }
    } else {
      // fp8: fp32 rows, 64 pairs at a time, rounded on the way out (the bf16
      // staging above needs registers this instantiation does not have)
#pragma unroll
      for (int hp = 0; hp < (kPB + 1) / 2; ++hp) {   // pairs 64*hp .. 64*hp+63
        constexpr int kHalfPairs = kPB == 1 ? 32 : 64;
#pragma unroll
        for (int pbl = 0; pbl < kHalfPairs / 32; ++pbl) {
          const int pb = 2 * hp + pbl;
          lds_u8* xrow = lds + (32 * pbl + (lane_x & 31)) * kXRow + (128 * wave + 4 * e_half) * 4;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              f32x4 v = f32x4{o[db * kPB + pb][4 * qq], o[db * kPB + pb][4 * qq + 1], o[db * kPB + pb][4 * qq + 2],
                              o[db * kPB + pb][4 * qq + 3]};
              *(lds_f32x4*)(xrow + (32 * db + 8 * qq) * 4) = v;
            }
        }
        lds_barrier();                              // the rows (and s_l, s_m) are in LDS
        // thread t: 16-byte chunk t % 128 of rows t / 128 + 2k
        const int c = e_tid & 127;
#pragma unroll 4
        for (int k = 0; k < kHalfPairs / 2; ++k) {
          const int r = (e_tid >> 7) + 2 * k;
          const int pair = 64 * hp + r;
          if (kPB != 4 && pair / hpw >= a.q_per_seq) continue;   // padding
          const int row_in_seq = (pair / hpw) * a.n_heads + hg * hpw + pair % hpw;
          const f32x4 v = *(const lds_f32x4*)(lds + r * kXRow + c * 16);
          if (!whole) {
            u32x2 pk2;
            pk2[0] = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
            pk2[1] = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
            *(u32x2*)(a.ws_o + (slot_row0 + row_in_seq) * kDc + 4 * c) = pk2;
          } else {
            const float l = s_l[pair];
            const float inv = l > 0.f ? 1.0f / l : 0.f;
            u32x2 pk2;
            pk2[0] = (uint32_t)f32_to_bf16_bits(v[0] * inv) | ((uint32_t)f32_to_bf16_bits(v[1] * inv) << 16);
            pk2[1] = (uint32_t)f32_to_bf16_bits(v[2] * inv) | ((uint32_t)f32_to_bf16_bits(v[3] * inv) << 16);
            *(u32x2*)(a.o_final + ((int64_t)b * rows_per_seq + row_in_seq) * kDc + 4 * c) = pk2;
          }
        }
        lds_barrier();                              // the staging rows are free again
      }
    }
    if (whole && e_tid < 32 * kPB && (kPB == 4 || e_tid / hpw < a.q_per_seq)) {
      const int pair = e_tid;
      const int row_in_seq = (pair / hpw) * a.n_heads + hg * hpw + pair % hpw;
      const float l = s_l[pair], m = s_m[pair];
      a.lse_final[(int64_t)b * rows_per_seq + row_in_seq] = l > 0.f ? (m + log2f(l)) * 0.69314718055994530942f : -INFINITY;
    }
    if (seq_end >= T1) break;
    lds_barrier();                             // s_l / s_m and the LDS stages are free again
    // next sequence holding tiles
    seq_start = seq_end;
    do {
      ++b;
    } while (tiles_of(seq_len(b)) == 0);
  }
}

}  // namespace

namespace {

// Pair blocks per work-group (kPB: 32 (query row, head) pairs each) and heads
// per work-group (hpw; grid.y = H / hpw head groups) for a shape: the fewest
// blocks that hold min(H, 128 / q_per_seq) heads x q_per_seq rows, kPB = 4
// only without padding.
bool decode576_shape(const mla_dims& d, int32_t q_per_seq, int* kpb, int* hpw) {
  if (q_per_seq <= 0) return false;
  for (int pb : {4, 2, 1}) {
    const int pairs = 32 * pb;
    if (pairs % q_per_seq != 0) continue;
    const int h = d.n_heads < pairs / q_per_seq ? d.n_heads : pairs / q_per_seq;
    if (d.n_heads % h != 0) continue;
    if (pb == 4 && h * q_per_seq != pairs) continue;      // kPB = 4 is built without padding
    if (pb > 1 && h * q_per_seq <= pairs / 2) continue;   // fewer blocks hold them
    *kpb = pb;
    *hpw = h;
    return true;
  }
  return false;
}

}  // namespace

bool decode576_supported(const mla_dims& d, int32_t q_per_seq) {
  if (d.d_c != 512 || d.d_rope != 64 || d.act_dtype != MLA_BF16) return false;
  if (d.cache_dtype != MLA_BF16 && d.cache_dtype != MLA_FP8_E4M3) return false;
  if (d.block_size % kTile != 0) return false;
  int kpb, hpw;
  return decode576_shape(d, q_per_seq, &kpb, &hpw);
}

int64_t decode576_default_units(const mla_dims& d, int32_t q_per_seq, int cu_count) {
  // one resident work-group per CU: the head groups of a unit (grid.y) run
  // side by side on one XCD and read its tiles through the same L2
  int kpb = 0, hpw = 0;
  if (!decode576_shape(d, q_per_seq, &kpb, &hpw)) return cu_count;
  const int groups = d.n_heads / hpw;
  return cu_count / groups > 0 ? cu_count / groups : 1;
}

mla_status launch_decode576(const mla_dims& d, const DecodePlan& plan, int32_t n_seq, int32_t q_per_seq,
                            const void* q_abs, const void* pool, int64_t n_pool_blocks, const int32_t* block_table,
                            int32_t max_blocks, const int32_t* seqlens, void* ws, void* o_lat, float* lse,
                            hipStream_t st) {
  Args a;
  a.q_abs = static_cast<const uint16_t*>(q_abs);
  a.pool = static_cast<const uint8_t*>(pool);
  a.o_final = static_cast<uint16_t*>(o_lat);
  a.lse_final = lse;
  a.ws_o = static_cast<uint16_t*>(ws);
  a.ws_stats = static_cast<float*>(ws) + plan.ws_stats_offset_floats;
  a.block_bytes = static_cast<int64_t>(mla_cache_block_bytes(&d));
  a.n_pool_blocks = n_pool_blocks;
  a.max_blocks = max_blocks;
  a.block_size = d.block_size;
  a.n_seq = n_seq;
  a.q_per_seq = q_per_seq;
  a.n_heads = d.n_heads;
  a.units = plan.n_splits;
  int kpb = 0, hpw = 0;
  if (!decode576_shape(d, q_per_seq, &kpb, &hpw)) return MLA_ERR_UNSUPPORTED;
  a.heads_per_wg = hpw;
  a.scale_log2 = d.softmax_scale * 1.4426950408889634f;
  dim3 grid(plan.n_splits, d.n_heads / hpw);
  const bool f8 = d.cache_dtype == MLA_FP8_E4M3;
  void (*kern)(Args, const int32_t*, const int32_t*) =
      f8 ? (kpb == 4 ? decode576_kernel<true, 4> : kpb == 2 ? decode576_kernel<true, 2> : decode576_kernel<true, 1>)
         : (kpb == 4 ? decode576_kernel<false, 4> : kpb == 2 ? decode576_kernel<false, 2> : decode576_kernel<false, 1>);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, a, block_table, seqlens);
  return launch_status();
}

}  // namespace mla
