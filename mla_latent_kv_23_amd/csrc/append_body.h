// The per-token body of the cache append, shared by the append kernel and
// the fused absorb + append kernel.
#pragma once

#include "mla_internal.h"

namespace mla {

// Append token n into the paged cache: [c_kv[n] | RoPE(k_rope[n], pos[n])]
// at the cache dtype (fp8: per-token scale amax / 448, RNE-saturated E4M3FN
// codes, bf16 rotated k_R).  Run by a whole 256-thread work-group; `red` is
// 256 floats of LDS.  A token with an invalid sequence, position or block
// entry is skipped.
template <typename T, bool kFp8>
__device__ __forceinline__ void append_token(int n, const T* __restrict__ c_kv, const T* __restrict__ k_rope,
                                             const int32_t* __restrict__ seq_id, const int32_t* __restrict__ pos,
                                             const int32_t* __restrict__ block_table, int n_seq, int max_blocks,
                                             uint8_t* __restrict__ pool, int64_t n_pool_blocks, int64_t block_bytes,
                                             int block_size, int d_c, int d_rope, const RopeFreqs& freqs,
                                             float* red) {
  const int sq = seq_id[n], p = pos[n];
  if (sq < 0 || sq >= n_seq || p < 0 || p / block_size >= max_blocks) return;
  const int32_t blk = block_table[static_cast<int64_t>(sq) * max_blocks + p / block_size];
  if (blk < 0 || blk >= n_pool_blocks) return;
  const int slot = p % block_size;
  uint8_t* base = pool + static_cast<int64_t>(blk) * block_bytes;
  const int64_t crow = static_cast<int64_t>(n) * d_c, krow = static_cast<int64_t>(n) * d_rope;
  if constexpr (!kFp8) {
    T* row = reinterpret_cast<T*>(base) + static_cast<int64_t>(slot) * (d_c + d_rope);
    for (int c = threadIdx.x; c < d_c; c += blockDim.x) row[c] = c_kv[crow + c];
    for (int i = threadIdx.x; i < d_rope / 2; i += blockDim.x) {
      float cs, sn, ox, oy;
      rope_cos_sin(p, freqs.inv_freq[i], &cs, &sn);
      rope_pair(Act<T>::ld(k_rope, krow + 2 * i), Act<T>::ld(k_rope, krow + 2 * i + 1), cs, sn, &ox, &oy);
      Act<T>::st(row, d_c + 2 * i, ox);
      Act<T>::st(row, d_c + 2 * i + 1, oy);
    }
  } else {
    // per-token amax -> scale = amax / 448 -> codes
    float amax = 0.f;
    for (int c = threadIdx.x; c < d_c; c += blockDim.x) amax = fmaxf(amax, fabsf(Act<T>::ld(c_kv, crow + c)));
    red[threadIdx.x] = amax;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
      if (threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
      __syncthreads();
    }
    amax = red[0];
    const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
    uint8_t* codes = base + static_cast<int64_t>(slot) * d_c;
    for (int c = threadIdx.x; c < d_c; c += blockDim.x) codes[c] = f32_to_e4m3fn(Act<T>::ld(c_kv, crow + c) / scale);
    if (threadIdx.x == 0) reinterpret_cast<float*>(base + static_cast<int64_t>(block_size) * d_c)[slot] = scale;
    uint16_t* kr = reinterpret_cast<uint16_t*>(base + static_cast<int64_t>(block_size) * d_c + 4 * block_size) +
                   static_cast<int64_t>(slot) * d_rope;
    for (int i = threadIdx.x; i < d_rope / 2; i += blockDim.x) {
      float cs, sn, ox, oy;
      rope_cos_sin(p, freqs.inv_freq[i], &cs, &sn);
      rope_pair(Act<T>::ld(k_rope, krow + 2 * i), Act<T>::ld(k_rope, krow + 2 * i + 1), cs, sn, &ox, &oy);
      kr[2 * i] = f32_to_bf16_bits(ox);
      kr[2 * i + 1] = f32_to_bf16_bits(oy);
    }
  }
}

}  // namespace mla
