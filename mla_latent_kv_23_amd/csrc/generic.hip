// Generic (any-dimension, any supported dtype) kernels of libmla.  These are
// straightforward scalar kernels: they serve small or unusual shapes (such as
// a 64-wide latent in float32) and every shape the tuned gfx950 kernels do not
// cover.  The tuned kernels live in their own files.
#include "append_body.h"
#include "mla_internal.h"

namespace mla {

// ----------------------------------------------------------------------------
// absorb: q_abs[t,s,:d_c] = sum_n q_nope[t,s,n] w_uk[s,n,:]; q_abs[t,s,d_c:] = RoPE(q_rope[t,s,:], pos[t])
// grid (n_tok, H), block 256.
// ----------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) absorb_generic_kernel(
    const T* __restrict__ q_nope, const T* __restrict__ q_rope, const int32_t* __restrict__ pos,
    const T* __restrict__ w_uk, T* __restrict__ q_abs, int H, int d_c, int d_rope, int d_nope,
    RopeFreqs freqs) {
  extern __shared__ float sh_q[];           // d_nope floats
  const int t = blockIdx.x, s = blockIdx.y;
  const int64_t row = static_cast<int64_t>(t) * H + s;
  for (int n = threadIdx.x; n < d_nope; n += blockDim.x) sh_q[n] = Act<T>::ld(q_nope, row * d_nope + n);
  __syncthreads();
  const int d_k = d_c + d_rope;
  const T* w = w_uk + static_cast<int64_t>(s) * d_nope * d_c;
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
    float acc = 0.f;
    for (int n = 0; n < d_nope; ++n) acc = fmaf(sh_q[n], Act<T>::ld(w, static_cast<int64_t>(n) * d_c + c), acc);
    Act<T>::st(q_abs, row * d_k + c, acc);
  }
  if (d_rope == 0) return;                  // no RoPE part: q_rope and pos may be null
  const int p = pos[t];
  for (int i = threadIdx.x; i < d_rope / 2; i += blockDim.x) {
    float cs, sn, ox, oy;
    rope_cos_sin(p, freqs.inv_freq[i], &cs, &sn);
    rope_pair(Act<T>::ld(q_rope, row * d_rope + 2 * i), Act<T>::ld(q_rope, row * d_rope + 2 * i + 1), cs, sn, &ox, &oy);
    Act<T>::st(q_abs, row * d_k + d_c + 2 * i, ox);
    Act<T>::st(q_abs, row * d_k + d_c + 2 * i + 1, oy);
  }
}

// ----------------------------------------------------------------------------
// append: one block per token (the body is in append_body.h).
// ----------------------------------------------------------------------------
template <typename T, bool kFp8>
__global__ void __launch_bounds__(256) append_generic_kernel(
    const T* __restrict__ c_kv, const T* __restrict__ k_rope, const int32_t* __restrict__ seq_id,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ block_table, int n_seq, int max_blocks,
    uint8_t* __restrict__ pool, int64_t n_pool_blocks, int64_t block_bytes, int block_size, int d_c,
    int d_rope, RopeFreqs freqs) {
  __shared__ float red[256];
  append_token<T, kFp8>(blockIdx.x, c_kv, k_rope, seq_id, pos, block_table, n_seq, max_blocks, pool, n_pool_blocks,
                        block_bytes, block_size, d_c, d_rope, freqs, red);
}

// ----------------------------------------------------------------------------
// decode: one block per (sequence, query row, head) and split k of the keys.
// grid (n_seq * q_per_seq * H, n_splits), block 256.  Split k covers key
// tokens [k*chunk, min((k+1)*chunk, p+1)), chunk = ceil(L / n_splits).
// ----------------------------------------------------------------------------
template <typename T, bool kFp8>
__global__ void __launch_bounds__(256) decode_generic_kernel(
    const T* __restrict__ q_abs, const uint8_t* __restrict__ pool, int64_t n_pool_blocks,
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ seqlens, int q_per_seq, int H, int d_c, int d_rope,
    int block_size, int64_t block_bytes, float scale, int n_splits, T* __restrict__ o_final,
    float* __restrict__ lse_final, float* __restrict__ ws_o, float* __restrict__ ws_stats) {
  extern __shared__ float sh[];             // q [d_c + d_rope] | p [256] | acc [d_c]
  const int d_k = d_c + d_rope;
  float* sh_q = sh;
  float* sh_p = sh + d_k;
  __shared__ float red[256];
  __shared__ float sh_m, sh_l, sh_alpha;
  const int row = blockIdx.x;                // ((b * q_per_seq) + j) * H + s
  const int s = row % H, j = (row / H) % q_per_seq, b = row / (H * q_per_seq);
  const int split = blockIdx.y;
  const int L = min(max(seqlens[b], 0), max_blocks * block_size);   // what the table can address
  const int p_q = L - q_per_seq + j;         // query position; sees tokens 0..p_q
  const int chunk = (L + n_splits - 1) / n_splits;
  const int t0 = split * chunk;
  const int t1 = min(t0 + chunk, p_q + 1);
  for (int k = threadIdx.x; k < d_k; k += blockDim.x) sh_q[k] = Act<T>::ld(q_abs, static_cast<int64_t>(row) * d_k + k);
  if (threadIdx.x == 0) { sh_m = -INFINITY; sh_l = 0.f; }
  // each thread owns latent dims c = tid + 256*r
  constexpr int kMaxPerThread = 16;          // d_c <= 4096
  float acc[kMaxPerThread];
#pragma unroll
  for (int r = 0; r < kMaxPerThread; ++r) acc[r] = 0.f;
  __syncthreads();
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_blocks;
  for (int tc = t0; tc < t1; tc += 256) {
    const int t = tc + threadIdx.x;
    float z = -INFINITY;
    if (t < t1 && bt[t / block_size] >= 0 && bt[t / block_size] < n_pool_blocks) {
      const uint8_t* blk = pool + static_cast<int64_t>(bt[t / block_size]) * block_bytes;
      const int slot = t % block_size;
      float dot = 0.f;
      if constexpr (!kFp8) {
        const T* kr = reinterpret_cast<const T*>(blk) + static_cast<int64_t>(slot) * d_k;
        for (int k = 0; k < d_k; ++k) dot = fmaf(sh_q[k], Act<T>::ld(kr, k), dot);
      } else {
        const uint8_t* codes = blk + static_cast<int64_t>(slot) * d_c;
        const float sc = reinterpret_cast<const float*>(blk + static_cast<int64_t>(block_size) * d_c)[slot];
        const uint16_t* kr = reinterpret_cast<const uint16_t*>(blk + static_cast<int64_t>(block_size) * d_c + 4 * block_size) +
                             static_cast<int64_t>(slot) * d_rope;
        float dc = 0.f;
        for (int k = 0; k < d_c; ++k) dc = fmaf(sh_q[k], e4m3fn_to_f32(codes[k]), dc);
        dot = dc * sc;
        for (int k = 0; k < d_rope; ++k) dot = fmaf(sh_q[d_c + k], bf16_bits_to_f32(kr[k]), dot);
      }
      z = dot * scale;
    }
    red[threadIdx.x] = z;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
      __syncthreads();
    }
    if (threadIdx.x == 0) {
      const float m_new = fmaxf(sh_m, red[0]);
      sh_alpha = (sh_m == -INFINITY) ? 0.f : expf(sh_m - m_new);
      sh_m = m_new;
    }
    __syncthreads();
    const float m = sh_m, alpha = sh_alpha;
    const float pt = (z == -INFINITY) ? 0.f : expf(z - m);
    sh_p[threadIdx.x] = pt;
    red[threadIdx.x] = pt;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) sh_l = sh_l * alpha + red[0];
    const int nt = min(256, t1 - tc);
#pragma unroll
    for (int r = 0; r < kMaxPerThread; ++r) {
      const int c = threadIdx.x + 256 * r;
      if (c < d_c) {
        float a = acc[r] * alpha;
        for (int u = 0; u < nt; ++u) {
          const int tt = tc + u;
          // padding entry or one outside the pool: weight 0, never read
          if (bt[tt / block_size] < 0 || bt[tt / block_size] >= n_pool_blocks) continue;
          const uint8_t* blk = pool + static_cast<int64_t>(bt[tt / block_size]) * block_bytes;
          const int slot = tt % block_size;
          float v;
          if constexpr (!kFp8) {
            v = Act<T>::ld(reinterpret_cast<const T*>(blk), static_cast<int64_t>(slot) * d_k + c);
          } else {
            v = e4m3fn_to_f32(blk[static_cast<int64_t>(slot) * d_c + c]) *
                reinterpret_cast<const float*>(blk + static_cast<int64_t>(block_size) * d_c)[slot];
          }
          a = fmaf(sh_p[u], v, a);
        }
        acc[r] = a;
      }
    }
    __syncthreads();
  }
  const float l = sh_l, m = sh_m;
  const bool final_out = (n_splits == 1);
  const float inv_l = l > 0.f ? 1.0f / l : 0.f;
  const float lse_v = l > 0.f ? m + logf(l) : -INFINITY;
#pragma unroll
  for (int r = 0; r < kMaxPerThread; ++r) {
    const int c = threadIdx.x + 256 * r;
    if (c < d_c) {
      const float v = acc[r] * inv_l;
      if (final_out) Act<T>::st(o_final, static_cast<int64_t>(row) * d_c + c, v);
      else ws_o[(static_cast<int64_t>(b) * n_splits + split) * q_per_seq * H * d_c + static_cast<int64_t>(j * H + s) * d_c + c] = v;
    }
  }
  if (threadIdx.x == 0) {
    if (final_out) lse_final[row] = lse_v;
    else ws_stats[((static_cast<int64_t>(b) * n_splits + split) * q_per_seq * H + j * H + s) * 2] = lse_v;
  }
}

// ----------------------------------------------------------------------------
// combine: one block per (sequence, query row, head); partial slots of
// sequence b are first..first+count-1 (see slot_range).  Normalised partials
// (kPerSequence) merge as lse = log sum e^(lse_k), o = sum e^(lse_k - lse) o_k;
// raw partials (kStreamTiles, log2 units) as M = max m_k, L = sum 2^(m_k-M) l_k,
// o = sum 2^(m_k - M) o_k / L, lse = (M + log2 L) ln 2.
// ----------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_stats, int n_splits, int q_per_seq, int H, int d_c,
    T* __restrict__ o_lat, float* __restrict__ lse) {
  // per-sequence splits (the generic decode's layout): slots b * n_splits + k,
  // normalised partials, stats[0] = lse_k; a split that saw no key has lse_k = -inf
  __shared__ float w_sh[kMaxCombineSlots];
  __shared__ float scale_sh, lse_sh;
  const int row = blockIdx.x;
  const int s = row % H, j = (row / H) % q_per_seq, b = row / (H * q_per_seq);
  const int64_t first = static_cast<int64_t>(b) * n_splits;
  const int count = min(n_splits, kMaxCombineSlots);
  const int64_t per_slot = static_cast<int64_t>(q_per_seq) * H;
  const int64_t rr = j * H + s;
  if (threadIdx.x == 0) {
    float m = -INFINITY;
    for (int k = 0; k < count; ++k) m = fmaxf(m, ws_stats[((first + k) * per_slot + rr) * 2]);
    const float msafe = (m == -INFINITY) ? 0.f : m;
    float tot = 0.f;
    for (int k = 0; k < count; ++k) {
      const float w = expf(ws_stats[((first + k) * per_slot + rr) * 2] - msafe);   // 0 for an empty split
      tot += w;
      w_sh[k] = w;
    }
    scale_sh = tot > 0.f ? 1.0f / tot : 0.f;
    lse_sh = (tot > 0.f) ? msafe + logf(tot) : -INFINITY;
  }
  __syncthreads();
  const float inv = scale_sh;
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
    float a = 0.f;
    for (int k = 0; k < count; ++k) {
      const float w = w_sh[k];
      if (w != 0.f) a = fmaf(w, ws_o[((first + k) * per_slot + rr) * d_c + c], a);
    }
    Act<T>::st(o_lat, static_cast<int64_t>(row) * d_c + c, a * inv);
  }
  if (threadIdx.x == 0) lse[row] = lse_sh;
}

// ----------------------------------------------------------------------------
// up-projection: out[t,s,v] = sum_c w_uv[s,v,c] o_lat[t,s,c], times
// sigmoid(gate[t,s,v]) when a gate is given; grid (n_tok, H), block 256
// ----------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) up_proj_generic_kernel(const T* __restrict__ o_lat, const T* __restrict__ w_uv,
                                                              const T* __restrict__ gate, T* __restrict__ out, int H,
                                                              int d_c, int d_v) {
  extern __shared__ float sh_o[];           // d_c
  const int t = blockIdx.x, s = blockIdx.y;
  const int64_t row = static_cast<int64_t>(t) * H + s;
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) sh_o[c] = Act<T>::ld(o_lat, row * d_c + c);
  __syncthreads();
  const T* w = w_uv + static_cast<int64_t>(s) * d_v * d_c;
  // one wave per output element at a time: lanes split the d_c reduction
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n_waves = blockDim.x >> 6;
  for (int v = wave; v < d_v; v += n_waves) {
    float a = 0.f;
    for (int c = lane; c < d_c; c += 64) a = fmaf(sh_o[c], Act<T>::ld(w, static_cast<int64_t>(v) * d_c + c), a);
    for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
    if (lane == 0) {
      if (gate) a *= sigmoid_f32(Act<T>::ld(gate, row * d_v + v));
      Act<T>::st(out, row * d_v + v, a);
    }
  }
}

// ----------------------------------------------------------------------------
// host launchers
// ----------------------------------------------------------------------------

mla_status launch_absorb_generic(const mla_dims& d, int32_t n_tok, const void* q_nope, const void* q_rope,
                                 const int32_t* pos, const void* w_uk, void* q_abs, hipStream_t st) {
  const RopeFreqs f = make_rope_freqs(d);
  dim3 grid(n_tok, d.n_heads);
  const size_t shm = sizeof(float) * d.d_nope;
  if (d.act_dtype == MLA_F32)
    hipLaunchKernelGGL(absorb_generic_kernel<float>, grid, dim3(256), shm, st, (const float*)q_nope,
                       (const float*)q_rope, pos, (const float*)w_uk, (float*)q_abs, d.n_heads, d.d_c,
                       d.d_rope, d.d_nope, f);
  else
    hipLaunchKernelGGL(absorb_generic_kernel<uint16_t>, grid, dim3(256), shm, st, (const uint16_t*)q_nope,
                       (const uint16_t*)q_rope, pos, (const uint16_t*)w_uk, (uint16_t*)q_abs, d.n_heads,
                       d.d_c, d.d_rope, d.d_nope, f);
  return launch_status();
}

mla_status launch_append_generic(const mla_dims& d, int32_t n_tok, const void* c_kv, const void* k_rope,
                                 const int32_t* seq_id, const int32_t* pos, const int32_t* block_table,
                                 int32_t n_seq, int32_t max_blocks, void* pool, int64_t n_pool_blocks,
                                 hipStream_t st) {
  const RopeFreqs f = make_rope_freqs(d);
  const int64_t bb = static_cast<int64_t>(mla_cache_block_bytes(&d));
  if (d.cache_dtype == MLA_F32)
    hipLaunchKernelGGL((append_generic_kernel<float, false>), dim3(n_tok), dim3(256), 0, st, (const float*)c_kv,
                       (const float*)k_rope, seq_id, pos, block_table, n_seq, max_blocks, (uint8_t*)pool,
                       n_pool_blocks, bb, d.block_size, d.d_c, d.d_rope, f);
  else if (d.cache_dtype == MLA_BF16)
    hipLaunchKernelGGL((append_generic_kernel<uint16_t, false>), dim3(n_tok), dim3(256), 0, st,
                       (const uint16_t*)c_kv, (const uint16_t*)k_rope, seq_id, pos, block_table, n_seq,
                       max_blocks, (uint8_t*)pool, n_pool_blocks, bb, d.block_size, d.d_c, d.d_rope, f);
  else
    hipLaunchKernelGGL((append_generic_kernel<uint16_t, true>), dim3(n_tok), dim3(256), 0, st,
                       (const uint16_t*)c_kv, (const uint16_t*)k_rope, seq_id, pos, block_table, n_seq,
                       max_blocks, (uint8_t*)pool, n_pool_blocks, bb, d.block_size, d.d_c, d.d_rope, f);
  return launch_status();
}

mla_status launch_decode_generic(const mla_dims& d, const DecodePlan& plan, int32_t n_seq, int32_t q_per_seq,
                                 const void* q_abs, const void* pool, int64_t n_pool_blocks,
                                 const int32_t* block_table, int32_t max_blocks, const int32_t* seqlens, void* ws,
                                 void* o_lat, float* lse, hipStream_t st) {
  const int64_t bb = static_cast<int64_t>(mla_cache_block_bytes(&d));
  dim3 grid(n_seq * q_per_seq * d.n_heads, plan.n_splits);
  const size_t shm = sizeof(float) * (d.d_c + d.d_rope + 256);
  float* ws_o = static_cast<float*>(ws);
  float* ws_stats = ws_o ? ws_o + plan.ws_stats_offset_floats : nullptr;
  if (d.cache_dtype == MLA_F32)
    hipLaunchKernelGGL((decode_generic_kernel<float, false>), grid, dim3(256), shm, st, (const float*)q_abs,
                       (const uint8_t*)pool, n_pool_blocks, block_table, max_blocks, seqlens, q_per_seq, d.n_heads, d.d_c,
                       d.d_rope, d.block_size, bb, d.softmax_scale, plan.n_splits, (float*)o_lat, lse, ws_o,
                       ws_stats);
  else if (d.cache_dtype == MLA_BF16)
    hipLaunchKernelGGL((decode_generic_kernel<uint16_t, false>), grid, dim3(256), shm, st,
                       (const uint16_t*)q_abs, (const uint8_t*)pool, n_pool_blocks, block_table, max_blocks, seqlens, q_per_seq,
                       d.n_heads, d.d_c, d.d_rope, d.block_size, bb, d.softmax_scale, plan.n_splits,
                       (uint16_t*)o_lat, lse, ws_o, ws_stats);
  else
    hipLaunchKernelGGL((decode_generic_kernel<uint16_t, true>), grid, dim3(256), shm, st,
                       (const uint16_t*)q_abs, (const uint8_t*)pool, n_pool_blocks, block_table, max_blocks, seqlens, q_per_seq,
                       d.n_heads, d.d_c, d.d_rope, d.block_size, bb, d.softmax_scale, plan.n_splits,
                       (uint16_t*)o_lat, lse, ws_o, ws_stats);
  return launch_status();
}

mla_status launch_combine(const mla_dims& d, const DecodePlan& plan, int32_t n_seq, int32_t q_per_seq,
                          const int32_t* seqlens, const void* ws, void* o_lat, float* lse, hipStream_t st) {
  if (plan.layout.mode == 1)   // only the tuned decode (bf16, d_c = 512) leaves this layout
    return launch_combine_stream(d, plan, n_seq, q_per_seq, seqlens, ws, o_lat, lse, st);
  const float* ws_o = static_cast<const float*>(ws);
  const float* ws_stats = ws_o + plan.ws_stats_offset_floats;
  dim3 grid(n_seq * q_per_seq * d.n_heads);
  if (d.act_dtype == MLA_F32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, st, ws_o, ws_stats, plan.n_splits, q_per_seq,
                       d.n_heads, d.d_c, (float*)o_lat, lse);
  else
    hipLaunchKernelGGL(combine_kernel<uint16_t>, grid, dim3(256), 0, st, ws_o, ws_stats, plan.n_splits, q_per_seq,
                       d.n_heads, d.d_c, (uint16_t*)o_lat, lse);
  return launch_status();
}

mla_status launch_up_proj_generic(const mla_dims& d, int32_t n_tok, const void* o_lat, const void* w_uv,
                                  const void* gate, void* out, hipStream_t st) {
  dim3 grid(n_tok, d.n_heads);
  const size_t shm = sizeof(float) * d.d_c;
  if (d.act_dtype == MLA_F32)
    hipLaunchKernelGGL(up_proj_generic_kernel<float>, grid, dim3(256), shm, st, (const float*)o_lat,
                       (const float*)w_uv, (const float*)gate, (float*)out, d.n_heads, d.d_c, d.d_v);
  else
    hipLaunchKernelGGL(up_proj_generic_kernel<uint16_t>, grid, dim3(256), shm, st, (const uint16_t*)o_lat,
                       (const uint16_t*)w_uv, (const uint16_t*)gate, (uint16_t*)out, d.n_heads, d.d_c, d.d_v);
  return launch_status();
}

}  // namespace mla
