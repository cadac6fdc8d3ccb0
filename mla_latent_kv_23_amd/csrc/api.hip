// C ABI of libmla: host-side validation, decode planning and dispatch.  Every
// entry point checks its arguments before launching anything and returns a
// status; no C++ exception crosses the boundary.
#include <cstdint>
#include <cmath>
#include <cstring>
#include <mutex>

#include "mla_internal.h"
#include "decode_latent576.h"

// Scratch of mla_decode_noalloc: the split partials and their statistics live
// in this array instead of a caller-provided workspace.  Each GPU the library
// runs on holds its own copy until the process ends.  In host code the name is
// only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress, once per device (mla::noalloc_scratch).
static __device__ __align__(256) uint8_t scratch[MLA_DECODE_NOALLOC_MAX_BYTES];

namespace mla {

RopeFreqs make_rope_freqs(const mla_dims& d) {
  RopeFreqs f;
  std::memset(&f, 0, sizeof(f));
  for (int i = 0; i < d.d_rope / 2; ++i)
    f.inv_freq[i] = std::pow(static_cast<double>(d.rope_base), -(2.0 * i) / static_cast<double>(d.d_rope));
  return f;
}

mla_status launch_status() { return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool dims_valid(const mla_dims* d) {
  if (!d) return false;
  if (d->n_heads <= 0 || d->d_c <= 0 || d->d_rope < 0 || (d->d_rope & 1) || d->d_nope <= 0 || d->d_v <= 0 ||
      d->block_size <= 0)
    return false;
  if (!(std::isfinite(d->softmax_scale) && d->softmax_scale > 0.f)) return false;
  if (d->d_rope > 0 && !(std::isfinite(d->rope_base) && d->rope_base > 0.f)) return false;
  if (d->act_dtype != MLA_F32 && d->act_dtype != MLA_BF16) return false;
  if (d->cache_dtype != MLA_F32 && d->cache_dtype != MLA_BF16 && d->cache_dtype != MLA_FP8_E4M3) return false;
  return true;
}

// dtype pairing and the size limits of the kernels
mla_status dims_supported(const mla_dims* d) {
  if (!dims_valid(d)) return MLA_ERR_INVALID_ARG;
  if (d->cache_dtype == MLA_F32 && d->act_dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (d->cache_dtype != MLA_F32 && d->act_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (d->d_rope / 2 > kMaxRopePairs) return MLA_ERR_UNSUPPORTED;
  if (d->d_c > 4096 || d->d_c + d->d_rope > 8192 || d->d_nope > 8192 || d->d_v > 65535) return MLA_ERR_UNSUPPORTED;
  if (d->n_heads > 65535) return MLA_ERR_UNSUPPORTED;
  if (d->cache_dtype == MLA_FP8_E4M3 && (d->d_c % 4) != 0) return MLA_ERR_UNSUPPORTED;  // fp32 scales stay aligned
  return MLA_OK;
}

// Whether the tuned gfx950 kernel handles these dims and this query count.
bool tuned_decode_applies(const mla_dims& d, int32_t q_per_seq) {
  return decode576_supported(d, q_per_seq);
}

DecodePlan make_plan(const mla_dims& d, int32_t n_seq, int32_t q_per_seq, int32_t max_blocks, int32_t num_splits) {
  DecodePlan p;
  std::memset(&p, 0, sizeof(p));
  const int64_t max_len = static_cast<int64_t>(max_blocks) * d.block_size;
  if (tuned_decode_applies(d, q_per_seq)) {
    p.kind = 1;
    const int64_t tiles_bound = static_cast<int64_t>(n_seq) * ((max_len + kDecodeTile - 1) / kDecodeTile);
    int64_t units = num_splits > 0 ? num_splits : decode576_default_units(d, q_per_seq, device_cu_count());
    if (units > tiles_bound) units = tiles_bound;
    if (units < 1) units = 1;
    p.n_splits = static_cast<int32_t>(units);
    p.layout.mode = 1;
    p.layout.n_splits = p.n_splits;
    p.layout.tile = kDecodeTile;
    p.layout.max_len = static_cast<int32_t>(max_len);
    p.n_slots = p.n_splits + n_seq;       // also the staging area of whole sequences
    p.needs_combine = p.n_splits > 1 ? 1 : 0;
  } else {
    p.kind = 0;
    int64_t s = num_splits;
    if (s <= 0) {
      const int64_t rows = static_cast<int64_t>(n_seq) * q_per_seq * d.n_heads;
      const int64_t want = (2LL * device_cu_count() + rows - 1) / rows;
      const int64_t cap = (max_len + 255) / 256;
      s = want < cap ? want : cap;
    }
    if (s > kMaxCombineSlots) s = kMaxCombineSlots;
    if (s < 1) s = 1;
    p.n_splits = static_cast<int32_t>(s);
    p.layout.mode = 0;
    p.layout.n_splits = p.n_splits;
    p.layout.tile = 0;
    p.layout.max_len = static_cast<int32_t>(max_len);
    p.n_slots = p.n_splits > 1 ? n_seq * p.n_splits : 0;
    p.needs_combine = p.n_splits > 1 ? 1 : 0;
  }
  const int64_t rows_per_slot = static_cast<int64_t>(q_per_seq) * d.n_heads;
  // partials: bf16 for the tuned decode's stream layout, fp32 otherwise
  p.ws_stats_offset_floats = static_cast<int64_t>(p.n_slots) * rows_per_slot * d.d_c / (p.layout.mode == 1 ? 2 : 1);
  p.ws_bytes =
      p.n_slots ? static_cast<size_t>(p.ws_stats_offset_floats + 2LL * p.n_slots * rows_per_slot) * sizeof(float) : 0;
  return p;
}

// The device address of `scratch` on the current device, looked up with that
// device current on its first use and kept per device.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

mla_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

mla_status check_decode_args(const mla_dims* d, int32_t n_seq, int32_t q_per_seq, int32_t max_blocks,
                             int32_t num_splits) {
  const mla_status s = dims_supported(d);
  if (s != MLA_OK) return s;
  if (n_seq <= 0 || q_per_seq <= 0 || max_blocks <= 0 || num_splits < 0) return MLA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks) * d->block_size > (1LL << 30)) return MLA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(n_seq) * q_per_seq * d->n_heads > (1LL << 31) - 1) return MLA_ERR_UNSUPPORTED;
  // the decode kernels index the 32-token key tiles of all sequences in 32 bits
  if (static_cast<int64_t>(n_seq) * ((static_cast<int64_t>(max_blocks) * d->block_size + 31) / 32) > (1LL << 31) - 1)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" {

size_t mla_cache_block_bytes(const mla_dims* d) {
  if (!dims_valid(d)) return 0;
  const size_t bs = static_cast<size_t>(d->block_size);
  switch (d->cache_dtype) {
    case MLA_F32: return bs * (d->d_c + d->d_rope) * 4;
    case MLA_BF16: return bs * (d->d_c + d->d_rope) * 2;
    case MLA_FP8_E4M3: return bs * d->d_c + bs * 4 + bs * d->d_rope * 2;
    default: return 0;
  }
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported dims or dtype combination";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

mla_status mla_absorb_q(const mla_dims* d, int32_t n_tok, const void* q_nope, const void* q_rope,
                        const int32_t* pos, const void* w_uk, void* q_abs, mla_stream_t stream) {
  const mla_status s = dims_supported(d);
  if (s != MLA_OK) return s;
  if (n_tok < 0) return MLA_ERR_INVALID_ARG;
  if (n_tok == 0) return MLA_OK;
  if (!q_nope || !w_uk || !q_abs || (d->d_rope > 0 && (!q_rope || !pos))) return MLA_ERR_INVALID_ARG;
  if (n_tok > 2147483647 / d->n_heads) return MLA_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (absorb_tuned_applies(*d) && aligned16(q_nope) && aligned16(w_uk) && aligned16(q_abs))
    return launch_absorb_tuned(*d, n_tok, q_nope, q_rope, pos, w_uk, q_abs, st);
  return launch_absorb_generic(*d, n_tok, q_nope, q_rope, pos, w_uk, q_abs, st);
}

mla_status mla_append_cache(const mla_dims* d, int32_t n_tok, const void* c_kv, const void* k_rope,
                            const int32_t* seq_id, const int32_t* pos, const int32_t* block_table, int32_t n_seq,
                            int32_t max_blocks, void* cache_pool, int64_t n_pool_blocks, mla_stream_t stream) {
  const mla_status s = dims_supported(d);
  if (s != MLA_OK) return s;
  if (n_tok < 0 || n_seq <= 0 || max_blocks <= 0 || n_pool_blocks <= 0) return MLA_ERR_INVALID_ARG;
  if (n_tok == 0) return MLA_OK;
  if (!c_kv || !seq_id || !pos || !block_table || !cache_pool || (d->d_rope > 0 && !k_rope))
    return MLA_ERR_INVALID_ARG;
  return launch_append_generic(*d, n_tok, c_kv, k_rope, seq_id, pos, block_table, n_seq, max_blocks, cache_pool,
                               n_pool_blocks, static_cast<hipStream_t>(stream));
}

mla_status mla_absorb_append(const mla_dims* d, int32_t n_q, const void* q_nope, const void* q_rope,
                             const int32_t* q_pos, const void* w_uk, void* q_abs, int32_t n_kv, const void* c_kv,
                             const void* k_rope, const int32_t* seq_id, const int32_t* pos,
                             const int32_t* block_table, int32_t n_seq, int32_t max_blocks, void* cache_pool,
                             int64_t n_pool_blocks, mla_stream_t stream) {
  const mla_status s = dims_supported(d);
  if (s != MLA_OK) return s;
  // the checks of mla_absorb_q and mla_append_cache, all before any launch
  if (n_q < 0 || n_kv < 0 || n_seq <= 0 || max_blocks <= 0 || n_pool_blocks <= 0) return MLA_ERR_INVALID_ARG;
  if (n_q > 0 && (!q_nope || !w_uk || !q_abs || (d->d_rope > 0 && (!q_rope || !q_pos)))) return MLA_ERR_INVALID_ARG;
  if (n_kv > 0 && (!c_kv || !seq_id || !pos || !block_table || !cache_pool || (d->d_rope > 0 && !k_rope)))
    return MLA_ERR_INVALID_ARG;
  if (n_q > 2147483647 / d->n_heads) return MLA_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (n_q > 0 && n_kv > 0 && absorb_tuned_applies(*d) && d->cache_dtype != MLA_F32 && aligned16(q_nope) &&
      aligned16(w_uk) && aligned16(q_abs) && (int64_t)d->n_heads * (d->d_c / 128) + n_kv <= 2147483647LL)
    return launch_absorb_append(*d, n_q, q_nope, q_rope, q_pos, w_uk, q_abs, n_kv, c_kv, k_rope, seq_id, pos,
                                block_table, n_seq, max_blocks, cache_pool, n_pool_blocks, st);
  // otherwise the two calls in turn
  mla_status r = MLA_OK;
  if (n_q > 0) {
    r = (absorb_tuned_applies(*d) && aligned16(q_nope) && aligned16(w_uk) && aligned16(q_abs))
            ? launch_absorb_tuned(*d, n_q, q_nope, q_rope, q_pos, w_uk, q_abs, st)
            : launch_absorb_generic(*d, n_q, q_nope, q_rope, q_pos, w_uk, q_abs, st);
    if (r != MLA_OK) return r;
  }
  if (n_kv > 0)
    r = launch_append_generic(*d, n_kv, c_kv, k_rope, seq_id, pos, block_table, n_seq, max_blocks, cache_pool,
                              n_pool_blocks, st);
  return r;
}

size_t mla_decode_workspace_bytes(const mla_dims* d, int32_t n_seq, int32_t q_per_seq, int32_t max_blocks,
                                  int32_t num_splits) {
  if (check_decode_args(d, n_seq, q_per_seq, max_blocks, num_splits) != MLA_OK) return 0;
  return make_plan(*d, n_seq, q_per_seq, max_blocks, num_splits).ws_bytes;
}

int32_t mla_decode_needs_combine(const mla_dims* d, int32_t n_seq, int32_t q_per_seq, int32_t max_blocks,
                                 int32_t num_splits) {
  if (check_decode_args(d, n_seq, q_per_seq, max_blocks, num_splits) != MLA_OK) return 0;
  return make_plan(*d, n_seq, q_per_seq, max_blocks, num_splits).needs_combine;
}

mla_status mla_decode(const mla_dims* d, int32_t n_seq, int32_t q_per_seq, const void* q_abs,
                      const void* cache_pool, int64_t n_pool_blocks, const int32_t* block_table, int32_t max_blocks,
                      const int32_t* cache_seqlens, int32_t num_splits, void* workspace, size_t workspace_bytes,
                      void* o_latent, float* lse, mla_stream_t stream) {
  const mla_status s = check_decode_args(d, n_seq, q_per_seq, max_blocks, num_splits);
  if (s != MLA_OK) return s;
  if (n_pool_blocks <= 0) return MLA_ERR_INVALID_ARG;
  if (!q_abs || !cache_pool || !block_table || !cache_seqlens || !o_latent || !lse) return MLA_ERR_INVALID_ARG;
  const DecodePlan plan = make_plan(*d, n_seq, q_per_seq, max_blocks, num_splits);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes)) return MLA_ERR_WORKSPACE;
  if (plan.ws_bytes > 0 && (reinterpret_cast<uintptr_t>(workspace) & 15)) return MLA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (plan.kind == 1) {
    if (!aligned16(q_abs) || !aligned16(cache_pool) || !aligned16(o_latent)) return MLA_ERR_INVALID_ARG;
    return launch_decode576(*d, plan, n_seq, q_per_seq, q_abs, cache_pool, n_pool_blocks, block_table, max_blocks,
                            cache_seqlens, workspace, o_latent, lse, st);
  }
  return launch_decode_generic(*d, plan, n_seq, q_per_seq, q_abs, cache_pool, n_pool_blocks, block_table, max_blocks,
                               cache_seqlens, plan.ws_bytes ? workspace : nullptr, o_latent, lse, st);
}

mla_status mla_decode_noalloc(const mla_dims* d, int32_t n_seq, int32_t q_per_seq, const void* q_abs,
                              const void* cache_pool, int64_t n_pool_blocks, const int32_t* block_table,
                              int32_t max_blocks, const int32_t* cache_seqlens, int32_t num_splits, void* o_latent,
                              float* lse, mla_stream_t stream) {
  const mla_status s = check_decode_args(d, n_seq, q_per_seq, max_blocks, num_splits);
  if (s != MLA_OK) return s;
  if (n_pool_blocks <= 0) return MLA_ERR_INVALID_ARG;
  if (!q_abs || !cache_pool || !block_table || !cache_seqlens || !o_latent || !lse) return MLA_ERR_INVALID_ARG;
  const DecodePlan plan = make_plan(*d, n_seq, q_per_seq, max_blocks, num_splits);
  if (plan.ws_bytes > static_cast<size_t>(MLA_DECODE_NOALLOC_MAX_BYTES)) return MLA_ERR_WORKSPACE;
  if (plan.kind == 1 && (!aligned16(q_abs) || !aligned16(cache_pool) || !aligned16(o_latent)))
    return MLA_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (plan.ws_bytes > 0) {
    const mla_status g = noalloc_scratch(&ws);
    if (g != MLA_OK) return g;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  mla_status r = plan.kind == 1 ? launch_decode576(*d, plan, n_seq, q_per_seq, q_abs, cache_pool, n_pool_blocks,
                                                   block_table, max_blocks, cache_seqlens, ws, o_latent, lse, st)
                                : launch_decode_generic(*d, plan, n_seq, q_per_seq, q_abs, cache_pool, n_pool_blocks,
                                                        block_table, max_blocks, cache_seqlens, ws, o_latent, lse, st);
  if (r == MLA_OK && plan.needs_combine)
    r = launch_combine(*d, plan, n_seq, q_per_seq, cache_seqlens, ws, o_latent, lse, st);
  return r;
}

mla_status mla_check_block_table(const int32_t* block_table, int32_t n_seq, int32_t max_blocks,
                                 const int32_t* cache_seqlens, int32_t block_size, int64_t n_pool_blocks,
                                 int64_t* first_bad) {
  auto fail = [&](int64_t where) {
    if (first_bad) *first_bad = where;
    return MLA_ERR_INVALID_ARG;
  };
  if (n_seq < 0 || max_blocks <= 0 || block_size <= 0 || n_pool_blocks <= 0) return fail(INT64_MIN);
  if (n_seq > 0 && (!block_table || !cache_seqlens)) return fail(INT64_MIN);
  const int64_t max_len = static_cast<int64_t>(max_blocks) * block_size;
  for (int32_t b = 0; b < n_seq; ++b) {
    const int64_t L = cache_seqlens[b];
    if (L < 0 || L > max_len) return fail(-static_cast<int64_t>(b) - 1);
    const int64_t used = (L + block_size - 1) / block_size;
    const int32_t* row = block_table + static_cast<int64_t>(b) * max_blocks;
    for (int64_t i = 0; i < used; ++i)
      if (row[i] < 0 || row[i] >= n_pool_blocks) return fail(static_cast<int64_t>(b) * max_blocks + i);
  }
  if (first_bad) *first_bad = 0;
  return MLA_OK;
}

mla_status mla_combine(const mla_dims* d, int32_t n_seq, int32_t q_per_seq, const int32_t* cache_seqlens,
                       int32_t max_blocks, int32_t num_splits, const void* workspace, size_t workspace_bytes,
                       void* o_latent, float* lse, mla_stream_t stream) {
  const mla_status s = check_decode_args(d, n_seq, q_per_seq, max_blocks, num_splits);
  if (s != MLA_OK) return s;
  if (!cache_seqlens || !o_latent || !lse) return MLA_ERR_INVALID_ARG;
  const DecodePlan plan = make_plan(*d, n_seq, q_per_seq, max_blocks, num_splits);
  if (!plan.needs_combine) return MLA_OK;
  if (!workspace || workspace_bytes < plan.ws_bytes) return MLA_ERR_WORKSPACE;
  return launch_combine(*d, plan, n_seq, q_per_seq, cache_seqlens, workspace, o_latent, lse,
                        static_cast<hipStream_t>(stream));
}

namespace {
mla_status up_proj_common(const mla_dims* d, int32_t n_tok, const void* o_latent, const void* w_uv,
                          const void* gate, void* out, mla_stream_t stream) {
  const mla_status s = dims_supported(d);
  if (s != MLA_OK) return s;
  if (n_tok < 0) return MLA_ERR_INVALID_ARG;
  if (n_tok == 0) return MLA_OK;
  if (!o_latent || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (n_tok > 2147483647 / d->n_heads) return MLA_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the tuned kernel reads the gate in 8-byte pieces
  if (up_proj_tuned_applies(*d) && aligned16(o_latent) && aligned16(w_uv) && aligned16(out) &&
      (!gate || aligned16(gate)))
    return launch_up_proj_tuned(*d, n_tok, o_latent, w_uv, gate, out, st);
  return launch_up_proj_generic(*d, n_tok, o_latent, w_uv, gate, out, st);
}
}  // namespace

mla_status mla_up_proj(const mla_dims* d, int32_t n_tok, const void* o_latent, const void* w_uv, void* out,
                       mla_stream_t stream) {
  return up_proj_common(d, n_tok, o_latent, w_uv, nullptr, out, stream);
}

mla_status mla_up_proj_gated(const mla_dims* d, int32_t n_tok, const void* o_latent, const void* w_uv,
                             const void* gate, void* out, mla_stream_t stream) {
  if (n_tok > 0 && !gate) return MLA_ERR_INVALID_ARG;
  return up_proj_common(d, n_tok, o_latent, w_uv, gate, out, stream);
}

mla_status mla_combine_up_proj(const mla_dims* d, int32_t n_seq, int32_t q_per_seq, const int32_t* cache_seqlens,
                               int32_t max_blocks, int32_t num_splits, const void* workspace, size_t workspace_bytes,
                               void* o_latent, int32_t write_latent, const void* w_uv, const void* gate, void* out,
                               float* lse, mla_stream_t stream) {
  const mla_status s = check_decode_args(d, n_seq, q_per_seq, max_blocks, num_splits);
  if (s != MLA_OK) return s;
  if (!cache_seqlens || !o_latent || !lse || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  const int32_t n_tok = n_seq * q_per_seq;
  if (n_tok > 2147483647 / d->n_heads) return MLA_ERR_UNSUPPORTED;
  const DecodePlan plan = make_plan(*d, n_seq, q_per_seq, max_blocks, num_splits);
  if (plan.needs_combine && (!workspace || workspace_bytes < plan.ws_bytes)) return MLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (plan.needs_combine && combine_up_proj_applies(*d, plan) && aligned16(o_latent) && aligned16(w_uv) &&
      aligned16(out) && aligned16(workspace) && (!gate || aligned16(gate)))
    return launch_combine_up_proj(*d, plan, n_seq, q_per_seq, cache_seqlens, workspace, o_latent,
                                  write_latent ? o_latent : nullptr, w_uv, gate, out, lse, st);
  // otherwise the two calls (their kernels), the merged rows through o_latent
  if (plan.needs_combine) {
    const mla_status c = launch_combine(*d, plan, n_seq, q_per_seq, cache_seqlens, workspace, o_latent, lse, st);
    if (c != MLA_OK) return c;
  }
  return up_proj_common(d, n_tok, o_latent, w_uv, gate, out, stream);
}

size_t mla_prefill_workspace_bytes(const mla_dims* d, int32_t total_tokens) {
  if (dims_supported(d) != MLA_OK || !prefill_supported(*d) || total_tokens < 0) return 0;
  return prefill_workspace_bytes(*d, total_tokens);
}

mla_status mla_prefill(const mla_dims* d, int32_t n_seq, const int32_t* cu_seqlens, int32_t total_tokens,
                       int32_t max_seqlen, const void* q_nope, const void* q_rope, const void* c_kv,
                       const void* k_rope, const void* w_uk, const void* w_uv, const void* gate, void* workspace,
                       size_t workspace_bytes, void* out, float* lse, mla_stream_t stream) {
  const mla_status s = dims_supported(d);
  if (s != MLA_OK) return s;
  if (!prefill_supported(*d)) return MLA_ERR_UNSUPPORTED;
  if (n_seq <= 0 || total_tokens < 0 || max_seqlen < 0) return MLA_ERR_INVALID_ARG;
  if (total_tokens == 0) return MLA_OK;
  if (!cu_seqlens || !q_nope || !q_rope || !c_kv || !k_rope || !w_uk || !w_uv || !out || !lse)
    return MLA_ERR_INVALID_ARG;
  if (max_seqlen == 0 || max_seqlen > total_tokens) return MLA_ERR_INVALID_ARG;
  // 32-bit index math inside the kernels: tokens x heads x 128 and the grid
  if (static_cast<int64_t>(total_tokens) * d->n_heads * 128 > 2147483647LL) return MLA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(n_seq) * d->n_heads * ((max_seqlen + 127) / 128) > 2147483647LL) return MLA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < prefill_workspace_bytes(*d, total_tokens)) return MLA_ERR_WORKSPACE;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(c_kv) || !aligned16(k_rope) || !aligned16(w_uk) ||
      !aligned16(w_uv) || !aligned16(workspace) || !aligned16(out) || (gate && !aligned16(gate)))
    return MLA_ERR_INVALID_ARG;
  return launch_prefill(*d, n_seq, cu_seqlens, total_tokens, max_seqlen, q_nope, q_rope, c_kv, k_rope, w_uk, w_uv,
                        gate, workspace, out, lse, static_cast<hipStream_t>(stream));
}

size_t mla_prefill_paged_workspace_bytes(const mla_dims* d, int32_t total_q, int32_t total_k) {
  if (dims_supported(d) != MLA_OK || !prefill_supported(*d) || d->cache_dtype == MLA_F32 || total_q < 0 ||
      total_k < 0)
    return 0;
  return prefill_paged_workspace_bytes(*d, total_q, total_k);
}

mla_status mla_prefill_paged(const mla_dims* d, int32_t n_seq, const int32_t* cu_q, int32_t total_q, int32_t max_q,
                             const int32_t* cu_k, int32_t total_k, const void* q_nope, const void* q_rope,
                             const void* cache_pool, int64_t n_pool_blocks, const int32_t* block_table,
                             int32_t max_blocks, const void* w_uk, const void* w_uv, const void* gate, void* workspace,
                             size_t workspace_bytes, void* out, float* lse, mla_stream_t stream) {
  const mla_status s = dims_supported(d);
  if (s != MLA_OK) return s;
  if (!prefill_supported(*d) || d->cache_dtype == MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (n_seq <= 0 || total_q < 0 || max_q < 0 || total_k < 0 || max_blocks <= 0 || n_pool_blocks <= 0)
    return MLA_ERR_INVALID_ARG;
  if (total_q == 0) return MLA_OK;
  if (!cu_q || !cu_k || !q_nope || !q_rope || !cache_pool || !block_table || !w_uk || !w_uv || !out || !lse)
    return MLA_ERR_INVALID_ARG;
  if (max_q == 0 || max_q > total_q || total_k < total_q) return MLA_ERR_INVALID_ARG;
  // 32-bit index math: key tokens x heads x 128, the grid, block-table rows and pool rows
  if (static_cast<int64_t>(total_k) * d->n_heads * 128 > 2147483647LL) return MLA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(n_seq) * d->n_heads * ((max_q + 127) / 128) > 2147483647LL) return MLA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(max_blocks) * d->block_size > 2147483647LL) return MLA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < prefill_paged_workspace_bytes(*d, total_q, total_k)) return MLA_ERR_WORKSPACE;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(cache_pool) || !aligned16(w_uk) || !aligned16(w_uv) ||
      !aligned16(workspace) || !aligned16(out) || (gate && !aligned16(gate)))
    return MLA_ERR_INVALID_ARG;
  return launch_prefill_paged(*d, n_seq, cu_q, total_q, max_q, cu_k, total_k, q_nope, q_rope, cache_pool,
                              n_pool_blocks, block_table, max_blocks, w_uk, w_uv, gate, workspace, out, lse,
                              static_cast<hipStream_t>(stream));
}

namespace {
// the upstream GEMMs: bf16, 16-byte rows, whole float4 pieces of the partials
// that never straddle an output segment (the segment widths are multiples of 4)
bool upstream_shape_ok(const mla_dims* d, int64_t K, int64_t N) {
  return d->act_dtype == MLA_BF16 && K >= 16 && K % 16 == 0 && N % 8 == 0 && d->d_c % 4 == 0 && d->d_rope % 4 == 0 &&
         d->d_nope % 4 == 0;
}
}  // namespace

size_t mla_project_down_workspace_bytes(const mla_dims* d, int32_t n_tok, int32_t d_model, int32_t d_cq) {
  if (dims_supported(d) != MLA_OK || n_tok < 0 || d_model <= 0 || d_cq < 0) return 0;
  if (!upstream_shape_ok(d, d_model, (int64_t)d_cq + d->d_c + d->d_rope) || d_cq % 4 != 0) return 0;
  return project_down_workspace_bytes(*d, n_tok, d_model, d_cq);
}

mla_status mla_project_down(const mla_dims* d, int32_t n_tok, int32_t d_model, int32_t d_cq, const void* h,
                            const void* w_down, const int32_t* seq_id, const int32_t* pos,
                            const int32_t* block_table, int32_t n_seq, int32_t max_blocks, void* cache_pool,
                            int64_t n_pool_blocks, void* c_q, void* workspace, size_t workspace_bytes,
                            mla_stream_t stream) {
  const mla_status s = dims_supported(d);
  if (s != MLA_OK) return s;
  if (n_tok < 0 || d_model <= 0 || d_cq < 0 || n_seq <= 0 || max_blocks <= 0 || n_pool_blocks <= 0)
    return MLA_ERR_INVALID_ARG;
  const int64_t N = (int64_t)d_cq + d->d_c + d->d_rope;
  if (!upstream_shape_ok(d, d_model, N) || d_cq % 4 != 0) return MLA_ERR_UNSUPPORTED;
  if (n_tok == 0) return MLA_OK;
  if (!h || !w_down || !seq_id || !pos || !block_table || !cache_pool || (d_cq > 0 && !c_q))
    return MLA_ERR_INVALID_ARG;
  // 32-bit index math: rows of h and W and the partials' token x feature
  if ((int64_t)n_tok * d_model > 2147483647LL || N * d_model > 2147483647LL || (int64_t)n_tok * N > 2147483647LL)
    return MLA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < project_down_workspace_bytes(*d, n_tok, d_model, d_cq))
    return MLA_ERR_WORKSPACE;
  if (!aligned16(h) || !aligned16(w_down) || !aligned16(workspace) || (d_cq > 0 && !aligned16(c_q)))
    return MLA_ERR_INVALID_ARG;
  return launch_project_down(*d, n_tok, d_model, d_cq, h, w_down, seq_id, pos, block_table, n_seq, max_blocks,
                             cache_pool, n_pool_blocks, c_q, workspace, static_cast<hipStream_t>(stream));
}

size_t mla_absorb_from_latent_workspace_bytes(const mla_dims* d, int32_t n_tok, int32_t d_cq) {
  if (dims_supported(d) != MLA_OK || n_tok < 0 || d_cq <= 0) return 0;
  if (!upstream_shape_ok(d, d_cq, (int64_t)d->n_heads * (d->d_nope + d->d_rope))) return 0;
  return absorb_from_latent_workspace_bytes(*d, n_tok, d_cq);
}

mla_status mla_absorb_from_latent(const mla_dims* d, int32_t n_tok, int32_t d_cq, const void* c_q,
                                  const void* w_uq, const int32_t* pos, const void* w_uk, void* q_abs,
                                  void* workspace, size_t workspace_bytes, mla_stream_t stream) {
  const mla_status s = dims_supported(d);
  if (s != MLA_OK) return s;
  if (n_tok < 0 || d_cq <= 0) return MLA_ERR_INVALID_ARG;
  const int64_t N = (int64_t)d->n_heads * (d->d_nope + d->d_rope);
  if (!upstream_shape_ok(d, d_cq, N)) return MLA_ERR_UNSUPPORTED;
  if (n_tok == 0) return MLA_OK;
  if (!c_q || !w_uq || !pos || !w_uk || !q_abs) return MLA_ERR_INVALID_ARG;
  if ((int64_t)n_tok * d_cq > 2147483647LL || N * d_cq > 2147483647LL || (int64_t)n_tok * N > 2147483647LL)
    return MLA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < absorb_from_latent_workspace_bytes(*d, n_tok, d_cq)) return MLA_ERR_WORKSPACE;
  if (!aligned16(c_q) || !aligned16(w_uq) || !aligned16(workspace)) return MLA_ERR_INVALID_ARG;
  return launch_absorb_from_latent(*d, n_tok, d_cq, c_q, w_uq, pos, w_uk, q_abs, workspace,
                                   static_cast<hipStream_t>(stream));
}

}  // extern "C"
