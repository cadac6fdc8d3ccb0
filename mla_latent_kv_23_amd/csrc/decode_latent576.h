// Tuned gfx950 kernels for the 512-wide latent + 64-wide RoPE key shape.
#pragma once

#include "mla_internal.h"

namespace mla {

constexpr int kDecodeTile = 32;   // key tokens per pipeline stage of the tuned decode kernel

bool decode576_supported(const mla_dims& d, int32_t q_per_seq);
int64_t decode576_default_units(const mla_dims& d, int32_t q_per_seq, int cu_count);
mla_status launch_decode576(const mla_dims& d, const DecodePlan& plan, int32_t n_seq, int32_t q_per_seq,
                            const void* q_abs, const void* pool, int64_t n_pool_blocks, const int32_t* block_table,
                            int32_t max_blocks, const int32_t* seqlens, void* ws, void* o_lat, float* lse,
                            hipStream_t st);

bool absorb_tuned_applies(const mla_dims& d);
mla_status launch_absorb_append(const mla_dims& d, int32_t n_q, const void* q_nope, const void* q_rope,
                                const int32_t* q_pos, const void* w_uk, void* q_abs, int32_t n_kv, const void* c_kv,
                                const void* k_rope, const int32_t* seq_id, const int32_t* pos,
                                const int32_t* block_table, int32_t n_seq, int32_t max_blocks, void* pool,
                                int64_t n_pool_blocks, hipStream_t st);
mla_status launch_absorb_tuned(const mla_dims& d, int32_t n_tok, const void* q_nope, const void* q_rope,
                               const int32_t* pos, const void* w_uk, void* q_abs, hipStream_t st);
bool up_proj_tuned_applies(const mla_dims& d);
mla_status launch_up_proj_tuned(const mla_dims& d, int32_t n_tok, const void* o_lat, const void* w_uv,
                                const void* gate, void* out, hipStream_t st);

}  // namespace mla
