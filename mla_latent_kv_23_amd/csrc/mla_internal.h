// Internal declarations of libmla: decode plans, the partial-slot layout the
// decode and combine kernels agree on, and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"
#include "mla_device.h"

namespace mla {

constexpr int kMaxCombineSlots = 1024;   // partial results merged per (sequence, row, head)

// Workspace: partial outputs o[slot][q_per_seq * H][d_c], then per-row
// statistics stats[slot][q_per_seq * H][2] (fp32).
//   kPerSequence partials are fp32 and normalised: o = sum p v / sum p,
//   stats[0] = lse.
//   kStreamTiles partials are bf16 and raw: o = sum 2^(z - m) v, stats =
//   (m, sum 2^(z - m)), with z the scaled score in log2 units (the statistics
//   carry the scale, so one more rounding of o only adds 2^-9 relative noise,
//   averaged over the pieces by the merge).
// Where the partial results of sequence b live in the workspace.
//   kPerSequence: n_splits slots per sequence, slots b*n_splits .. +n_splits-1,
//                 split k covers keys [k*ceil(L/n), (k+1)*ceil(L/n)).
//   kStreamTiles: the key tiles of all sequences are laid end to end (sequence
//                 major, ceil(L_b / tile) tiles each) and cut into n_units equal
//                 runs; unit w handles tiles [floor(w*N/G), floor((w+1)*N/G)).
//                 The piece of sequence b done by unit w has slot w + b (unique
//                 because both indices only grow along the tile order).  A
//                 sequence that lies inside one unit gets its final output
//                 written directly and has no slots.
struct SplitLayout {
  int32_t mode;      // 0 = kPerSequence, 1 = kStreamTiles
  int32_t n_splits;  // kPerSequence: splits per sequence; kStreamTiles: units G
  int32_t tile;      // kStreamTiles: tokens per tile
  int32_t max_len;   // lengths are clamped to [0, max_len] (what the block table addresses)
};

struct DecodePlan {
  int32_t kind;                  // 0 = generic kernel, 1 = tuned gfx950 latent-576 kernel
  int32_t n_splits;              // generic: splits per sequence; tuned: work units
  int32_t n_slots;               // partial slots in the workspace (0 = none)
  int32_t needs_combine;         // partials are written (combine has work)
  int64_t ws_stats_offset_floats;  // per-row statistics start here (floats from workspace start)
  size_t ws_bytes;               // workspace bytes needed
  SplitLayout layout;
};

// Unit w of G over N tiles: first tile floor(w*N/G).
__host__ __device__ __forceinline__ int64_t unit_first_tile(int64_t w, int64_t N, int64_t G) { return w * N / G; }
// The unit that holds tile T.
__host__ __device__ __forceinline__ int64_t unit_of_tile(int64_t T, int64_t N, int64_t G) {
  return ((T + 1) * G - 1) / N;
}


RopeFreqs make_rope_freqs(const mla_dims& d);
mla_status launch_status();
int device_cu_count();

mla_status launch_absorb_generic(const mla_dims& d, int32_t n_tok, const void* q_nope, const void* q_rope,
                                 const int32_t* pos, const void* w_uk, void* q_abs, hipStream_t st);
mla_status launch_append_generic(const mla_dims& d, int32_t n_tok, const void* c_kv, const void* k_rope,
                                 const int32_t* seq_id, const int32_t* pos, const int32_t* block_table,
                                 int32_t n_seq, int32_t max_blocks, void* pool, int64_t n_pool_blocks,
                                 hipStream_t st);
mla_status launch_decode_generic(const mla_dims& d, const DecodePlan& plan, int32_t n_seq, int32_t q_per_seq,
                                 const void* q_abs, const void* pool, int64_t n_pool_blocks,
                                 const int32_t* block_table, int32_t max_blocks, const int32_t* seqlens, void* ws,
                                 void* o_lat, float* lse, hipStream_t st);
mla_status launch_combine(const mla_dims& d, const DecodePlan& plan, int32_t n_seq, int32_t q_per_seq,
                          const int32_t* seqlens, const void* ws, void* o_lat, float* lse, hipStream_t st);
mla_status launch_combine_stream(const mla_dims& d, const DecodePlan& plan, int32_t n_seq, int32_t q_per_seq,
                                 const int32_t* seqlens, const void* ws, void* o_lat, float* lse, hipStream_t st);
bool combine_up_proj_applies(const mla_dims& d, const DecodePlan& plan);
mla_status launch_combine_up_proj(const mla_dims& d, const DecodePlan& plan, int32_t n_seq, int32_t q_per_seq,
                                  const int32_t* seqlens, const void* ws, const void* o_lat, void* o_lat_out,
                                  const void* w_uv, const void* gate, void* out, float* lse, hipStream_t st);
bool prefill_supported(const mla_dims& d);
size_t prefill_workspace_bytes(const mla_dims& d, int64_t total_tokens);
size_t prefill_paged_workspace_bytes(const mla_dims& d, int64_t total_q, int64_t total_k);
mla_status launch_prefill(const mla_dims& d, int32_t n_seq, const int32_t* cu_seqlens, int32_t total_tokens,
                          int32_t max_seqlen, const void* q_nope, const void* q_rope, const void* c_kv,
                          const void* k_rope, const void* w_uk, const void* w_uv, const void* gate, void* ws,
                          void* out, float* lse, hipStream_t st);
mla_status launch_prefill_paged(const mla_dims& d, int32_t n_seq, const int32_t* cu_q, int32_t total_q, int32_t max_q,
                                const int32_t* cu_k, int32_t total_k, const void* q_nope, const void* q_rope,
                                const void* cache_pool, int64_t n_pool_blocks, const int32_t* block_table,
                                int32_t max_blocks,
                                const void* w_uk, const void* w_uv, const void* gate, void* ws, void* out, float* lse,
                                hipStream_t st);
size_t project_down_workspace_bytes(const mla_dims& d, int64_t n_tok, int64_t d_model, int64_t d_cq);
mla_status launch_project_down(const mla_dims& d, int32_t n_tok, int32_t d_model, int32_t d_cq, const void* h,
                               const void* w_down, const int32_t* seq_id, const int32_t* pos,
                               const int32_t* block_table, int32_t n_seq, int32_t max_blocks, void* pool,
                               int64_t n_pool_blocks, void* c_q, void* ws, hipStream_t st);
size_t absorb_from_latent_workspace_bytes(const mla_dims& d, int64_t n_tok, int64_t d_cq);
mla_status launch_absorb_from_latent(const mla_dims& d, int32_t n_tok, int32_t d_cq, const void* c_q,
                                     const void* w_uq, const int32_t* pos, const void* w_uk, void* q_abs, void* ws,
                                     hipStream_t st);
mla_status launch_up_proj_generic(const mla_dims& d, int32_t n_tok, const void* o_lat, const void* w_uv,
                                  const void* gate, void* out, hipStream_t st);

}  // namespace mla
