// Element-wise and bookkeeping kernels of librwkv7: row validation, embedding
// + LN0, the fused residual-fold + LayerNorm + token-shift mix, slot reset,
// weight packing, the sparse ReLU^2 channel-mix value, and the penalised
// greedy selection.
#include "launch.h"

#include <float.h>
#include <limits.h>

// ============================================================== validation
// One workgroup.  Rows (n_rows > 0): checks every row's slot (range,
// duplicates) and token (range), writes sanitized copies, bumps each valid
// slot's counter (decode steps do this inside k_embed_rows instead, one
// workgroup per row).  Prefill: checks tokens and bumps the slot's counter
// by n_tok.
// Rows whose slot repeats an earlier row's slot are dropped (the first
// occurrence keeps it).  The slot list is scanned from LDS when it fits.
constexpr int VALIDATE_LDS_ROWS = 4096;
__global__ __launch_bounds__(256) void k_validate(ValidateArgs a) {
  __shared__ int s_slot[VALIDATE_LDS_ROWS];
  const bool in_lds = a.n_rows <= VALIDATE_LDS_ROWS;
  if (in_lds) {
    for (int b = threadIdx.x; b < a.n_rows; b += 256) s_slot[b] = a.slot_idx[b];
    __syncthreads();
  }
  const int* list = in_lds ? s_slot : a.slot_idx;
  uint32_t bits = 0;
  for (int b = threadIdx.x; b < a.n_rows; b += 256) {
    const int s = list[b];
    int out = s;
    if (s < 0 || (int64_t)s >= a.n_slots) {
      bits |= ERRB_SLOT_RANGE;
      out = -1;
    } else {
      for (int j = 0; j < b; ++j)
        if (list[j] == s) {
          bits |= ERRB_SLOT_DUP;
          out = -1;
          break;
        }
    }
    a.slots_out[b] = out;
    if (out >= 0 && a.counters) a.counters[out] += 1;
  }
  for (int t = threadIdx.x; t < a.n_tok; t += 256) {
    int tok = a.tokens[t];
    if (tok < 0 || tok >= a.vocab) {
      bits |= ERRB_TOKEN_RANGE;
      tok = 0;
    }
    a.tok_out[t] = tok;
  }
  if (a.n_rows == 0 && threadIdx.x == 0 && a.counters && a.seq_slot >= 0)
    a.counters[a.seq_slot] += a.n_tok;
  for (int i = threadIdx.x; i < a.n_zero; i += 256) a.zero[i] = 0u;
  if (bits) set_err(a.err, bits);
}

hipError_t launch_validate(const ValidateArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_validate, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

__global__ void k_commit_shift(CommitArgs a) {
  const int b = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int slot = a.slots[b];
  if (c < a.C && slot >= 0 && slot < a.n_slots)
    a.pool[(long)slot * a.slot_stride + a.shift_off + c] = a.u[(long)b * a.C + c];
}

hipError_t launch_commit_shift(const CommitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_commit_shift, dim3((a.C + 255) / 256, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ============================================================== LayerNorm helpers
// Per-thread slice: elements c = threadIdx.x + 256*e, e < C/256 (<= 16).
template <int NE>
RW_DEV void ln_rows(const float* v, float* mean_out, float* rstd_out, float* red) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) s += v[e];
  const float C = 256.0f * NE;
  const float mean = block_sum_256(s, red) / C;
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const float d = v[e] - mean;
    q += d * d;
  }
  const float var = block_sum_256(q, red + 4) / C;
  *mean_out = mean;
  *rstd_out = 1.0f / sqrtf(var + 1e-5f);
}

// ============================================================== embedding
template <int NE>
__global__ __launch_bounds__(256) void k_embed(EmbedArgs a) {
  __shared__ float red[8];
  const int r = blockIdx.x;
  const int tok = a.tok[r];
  const half_t* e = a.emb + (long)tok * a.C;
  float v[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) v[i] = (float)e[threadIdx.x + 256 * i];
  float mean, rstd;
  ln_rows<NE>(v, &mean, &rstd, red);
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int c = threadIdx.x + 256 * i;
    a.x[(long)r * a.C + c] = (v[i] - mean) * rstd * a.g[c] + a.b[c];
  }
}

#define NE_DISPATCH(C, KERNEL, ...)                                                  \
  switch ((C) / 256) {                                                                \
    case 1: hipLaunchKernelGGL(KERNEL<1>, __VA_ARGS__); break;                        \
    case 2: hipLaunchKernelGGL(KERNEL<2>, __VA_ARGS__); break;                        \
    case 4: hipLaunchKernelGGL(KERNEL<4>, __VA_ARGS__); break;                        \
    case 8: hipLaunchKernelGGL(KERNEL<8>, __VA_ARGS__); break;                        \
    case 10: hipLaunchKernelGGL(KERNEL<10>, __VA_ARGS__); break;                       \
    case 12: hipLaunchKernelGGL(KERNEL<12>, __VA_ARGS__); break;                       \
    case 16: hipLaunchKernelGGL(KERNEL<16>, __VA_ARGS__); break;                       \
    default: return hipErrorInvalidValue;                                             \
  }

hipError_t launch_embed(const EmbedArgs& a, hipStream_t st) {
  if (a.C % 256) return hipErrorInvalidValue;
  NE_DISPATCH(a.C, k_embed, dim3(a.R), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Decode rows in one launch: workgroup r checks row r's slot (range; a slot
// listed by an earlier row drops this row, so the first occurrence keeps it)
// and token, writes their sanitized copies, bumps the slot's counter, and
// embeds the token with LN0 -- what k_validate and k_embed do, with the
// earlier-row comparisons spread over the workgroup's threads.
template <int NE>
__global__ __launch_bounds__(256) void k_embed_rows(ValidateArgs v, EmbedArgs a) {
  __shared__ float red[8];
  __shared__ int s_dup;
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  if (t == 0) s_dup = 0;
  __syncthreads();
  const int s = v.slot_idx[r];
  const bool in_range = s >= 0 && (int64_t)s < v.n_slots;
  if (in_range)
    for (int j = t; j < r; j += 256)
      if (v.slot_idx[j] == s) s_dup = 1;   // any writer: the value is the same
  __syncthreads();
  int tok = v.tokens[r];
  const bool tok_ok = tok >= 0 && tok < v.vocab;
  if (!tok_ok) tok = 0;
  if (t == 0) {
    uint32_t bits = 0;
    int out = s;
    if (!in_range) {
      bits |= ERRB_SLOT_RANGE;
      out = -1;
    } else if (s_dup) {
      bits |= ERRB_SLOT_DUP;
      out = -1;
    }
    if (!tok_ok) bits |= ERRB_TOKEN_RANGE;
    v.slots_out[r] = out;
    v.tok_out[r] = tok;
    if (out >= 0 && v.counters) v.counters[out] += 1;
    if (bits) set_err(v.err, bits);
  }
  const half_t* e = a.emb + (long)tok * a.C;
  float x[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) x[i] = (float)e[t + 256 * i];
  float mean, rstd;
  ln_rows<NE>(x, &mean, &rstd, red);
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int c = t + 256 * i;
    a.x[(long)r * a.C + c] = (x[i] - mean) * rstd * a.g[c] + a.b[c];
  }
}

hipError_t launch_embed_rows(const ValidateArgs& v, const EmbedArgs& a, hipStream_t st) {
  if (a.C % 256 || v.n_rows != a.R || v.n_tok != a.R || v.n_zero) return hipErrorInvalidValue;
  NE_DISPATCH(a.C, k_embed_rows, dim3(a.R), dim3(256), 0, st, v, a);
  return hipGetLastError();
}

// ============================================================== LN + token-shift mix
// One workgroup per row.  Every global load the row needs (x, partial sums,
// LayerNorm weights, the stored shift or the previous token's row, and all
// nq mixing vectors) is issued before the first reduction barrier, so a row
// costs one memory round trip.
// Row access of k_ln_mix: with NE even, element i of thread t is column
// 2t + 512 (i / 2) + i % 2, so every access moves two adjacent columns (one
// 8-byte load or store); with NE odd, column t + 256 i.
template <int NE>
RW_DEV int lnm_col(int t, int i) {
  return NE % 2 == 0 ? 2 * t + 512 * (i >> 1) + (i & 1) : t + 256 * i;
}
template <int NE>
RW_DEV void lnm_load(const float* p, float (&d)[NE], int t) {
  if constexpr (NE % 2 == 0) {
#pragma unroll
    for (int k = 0; k < NE / 2; ++k) {
      const float2 x = *reinterpret_cast<const float2*>(p + 2 * t + 512 * k);
      d[2 * k] = x.x;
      d[2 * k + 1] = x.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NE; ++i) d[i] = p[t + 256 * i];
  }
}
template <int NE>
RW_DEV void lnm_store(float* p, const float (&v)[NE], int t) {
  if constexpr (NE % 2 == 0) {
#pragma unroll
    for (int k = 0; k < NE / 2; ++k) *reinterpret_cast<float2*>(p + 2 * t + 512 * k) = make_float2(v[2 * k], v[2 * k + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < NE; ++i) p[t + 256 * i] = v[i];
  }
}
// Column blocks: a row's units (512-column pairs for NE even, 256-column
// slices for NE odd) are dealt round robin to the workgroups of the row;
// bit u of `own` is set for the units this workgroup loads and stores.
template <int NE>
RW_DEV constexpr int lnm_units() {
  return NE % 2 == 0 ? NE / 2 : NE;
}
template <int NE>
RW_DEV void lnm_load_own(const float* p, float (&d)[NE], int t, uint32_t own) {
  if constexpr (NE % 2 == 0) {
#pragma unroll
    for (int k = 0; k < NE / 2; ++k) {
      float2 x = make_float2(0.0f, 0.0f);
      if ((own >> k) & 1u) x = *reinterpret_cast<const float2*>(p + 2 * t + 512 * k);
      d[2 * k] = x.x;
      d[2 * k + 1] = x.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NE; ++i) d[i] = ((own >> i) & 1u) ? p[t + 256 * i] : 0.0f;
  }
}
template <int NE>
RW_DEV void lnm_store_own(float* p, const float (&v)[NE], int t, uint32_t own) {
  if constexpr (NE % 2 == 0) {
#pragma unroll
    for (int k = 0; k < NE / 2; ++k)
      if ((own >> k) & 1u) *reinterpret_cast<float2*>(p + 2 * t + 512 * k) = make_float2(v[2 * k], v[2 * k + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < NE; ++i)
      if ((own >> i) & 1u) p[t + 256 * i] = v[i];
  }
}
template <int NE>
RW_DEV void lnm_store_f16_own(half_t* p, const float (&v)[NE], int t, uint32_t own) {
  if constexpr (NE % 2 == 0) {
#pragma unroll
    for (int k = 0; k < NE / 2; ++k) {
      if (!((own >> k) & 1u)) continue;
      half2v h;
      h[0] = (half_t)v[2 * k];
      h[1] = (half_t)v[2 * k + 1];
      *reinterpret_cast<half2v*>(p + 2 * t + 512 * k) = h;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NE; ++i)
      if ((own >> i) & 1u) p[t + 256 * i] = (half_t)v[i];
  }
}

// LATE: the mixing vectors are loaded after the statistics, so they are not
// live across the reductions (fewer registers, more workgroups per CU; the
// sequence path, where rows fill the CUs several times over)
template <int NE, bool LATE = false>
__global__ __launch_bounds__(256) void k_ln_mix(LnMixArgs a) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  const int C = a.C;
  const int t = threadIdx.x;
  // column block blockIdx.y of gridDim.y: every block of a row reads the
  // whole row (and its partials) for the statistics, and loads and writes
  // only its own units of everything else
  uint32_t own = 0;
  for (int u = blockIdx.y; u < lnm_units<NE>(); u += gridDim.y) own |= 1u << u;
  if (a.cp_n && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = t; i < a.cp_n; i += 256) a.cp_dst[i] = a.cp_src[i];
  float v[NE], gv[NE], bv[NE], pv[NE], mu[6][NE];
  float* xr = a.x + (long)r * C;
  lnm_load<NE>(xr, v, t);
  lnm_load_own<NE>(a.g, gv, t, own);
  lnm_load_own<NE>(a.b, bv, t, own);
  const float* sh_in = nullptr;      // stored shift to mix with (decode / first token)
  float* sh_out = nullptr;           // where the new shift goes (decode)
  if (a.mode == LNMIX_DECODE) {
    const int slot = a.slots[r];
    if (slot >= 0 && slot < a.n_slots) {
      sh_out = a.pool + (long)slot * a.slot_stride + a.shift_off;
      sh_in = sh_out;
    }
  } else if (a.mode == LNMIX_SEQ && r == 0) {
    sh_in = a.pool + (long)a.seq_slot * a.slot_stride + a.shift_off;
  }
  const bool prev_row = a.mode == LNMIX_SEQ && r > 0;   // LayerNorm of the previous token
  const float* xp = a.x + (long)(r - 1) * C;
  if (sh_in) {
    lnm_load_own<NE>(sh_in, pv, t, own);
  } else if (prev_row) {
    lnm_load<NE>(xp, pv, t);
  } else {
#pragma unroll
    for (int i = 0; i < NE; ++i) pv[i] = 0.0f;
  }
  if (prev_row && a.nparts > 0) {
    // the previous row's residual with its partials folded in, computed the
    // same way as that row's own workgroup does (which writes it to x_out)
    float acc[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) acc[i] = 0.0f;
    const long rs = (long)a.R * C;
    const float* p = a.parts + (long)(r - 1) * C;
    for (int s = 0; s < a.nparts; ++s) {
      float q[NE];
      lnm_load<NE>(p + s * rs, q, t);
#pragma unroll
      for (int i = 0; i < NE; ++i) acc[i] += q[i];
    }
#pragma unroll
    for (int i = 0; i < NE; ++i) pv[i] += acc[i];
  }
  auto load_mu = [&]() {
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      if (q < a.nq && a.mu) {
        lnm_load_own<NE>(a.mu + (long)q * C, mu[q], t, own);
      } else {
#pragma unroll
        for (int i = 0; i < NE; ++i) mu[q][i] = 0.0f;
      }
    }
  };
  if constexpr (!LATE) load_mu();
  if (a.nparts > 0) {
    // x += (sum of the split-K partials of the residual projection, in range
    // order): the same arithmetic as the GEMM's own reduction pass
    // loads four ranges at a time (one memory round trip per four), adds in order
    float acc[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) acc[i] = 0.0f;
    const long rs = (long)a.R * C;   // floats between ranges
    const float* p = a.parts + (long)r * C;
    int s = 0;
    for (; s + 4 <= a.nparts; s += 4) {
      float q[4][NE];
#pragma unroll
      for (int j = 0; j < 4; ++j) lnm_load<NE>(p + (s + j) * rs, q[j], t);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < NE; ++i) acc[i] += q[j][i];
    }
    for (; s < a.nparts; ++s) {
      float q[NE];
      lnm_load<NE>(p + s * rs, q, t);
#pragma unroll
      for (int i = 0; i < NE; ++i) acc[i] += q[i];
    }
#pragma unroll
    for (int i = 0; i < NE; ++i) v[i] += acc[i];
    lnm_store_own<NE>(a.x_out ? a.x_out + (long)r * C : xr, v, t, own);
  }

  float mean, rstd;
  ln_rows<NE>(v, &mean, &rstd, red);
  if constexpr (LATE) load_mu();
  float u[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) u[i] = (v[i] - mean) * rstd * gv[i] + bv[i];
  if (prev_row) {
    float m2, rs2;
    ln_rows<NE>(pv, &m2, &rs2, red + 8);
#pragma unroll
    for (int i = 0; i < NE; ++i) pv[i] = (pv[i] - m2) * rs2 * gv[i] + bv[i];
  } else if (a.mode == LNMIX_PLAIN) {
#pragma unroll
    for (int i = 0; i < NE; ++i) pv[i] = u[i];
  }
  if (sh_out) lnm_store_own<NE>(sh_out, u, t, own);
  if (a.mode == LNMIX_SEQ && r == a.R - 1) lnm_store<NE>(a.shift_tmp, u, t);

#pragma unroll
  for (int q = 0; q < 6; ++q) {
    if (q >= a.nq) break;
    float o[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) o[i] = u[i] + (pv[i] - u[i]) * mu[q][i];
    const long off = q * a.out_q_stride + (long)r * C;
    if (a.out_f16)
      lnm_store_f16_own<NE>((half_t*)a.out + off, o, t, own);
    else
      lnm_store_own<NE>((float*)a.out + off, o, t, own);
  }
}

hipError_t launch_ln_mix(const LnMixArgs& a, hipStream_t st) {
  if (a.C % 256) return hipErrorInvalidValue;
  if (a.nq < 1 || a.nq > 6) return hipErrorInvalidValue;
  if (a.mode == LNMIX_SEQ && a.nparts && (!a.x_out || a.x_out == a.x)) return hipErrorInvalidValue;
  if (a.cp_n < 0 || (a.cp_n && (!a.cp_src || !a.cp_dst || a.cp_src == a.shift_tmp))) return hipErrorInvalidValue;
  // column blocks: not in sequence mode (a row also reads the previous row),
  // and with partials only into another buffer (the blocks of a row read
  // the whole residual row while its other blocks write theirs)
  const int units = (a.C / 256) % 2 == 0 ? a.C / 512 : a.C / 256;
  if (a.ncb < 1 || a.ncb > units) return hipErrorInvalidValue;
  if (a.ncb > 1 && (a.mode == LNMIX_SEQ || (a.nparts && (!a.x_out || a.x_out == a.x))))
    return hipErrorInvalidValue;
  if (a.mode == LNMIX_SEQ) {
    switch (a.C / 256) {
#define X(n) case n: hipLaunchKernelGGL((k_ln_mix<n, true>), dim3(a.R, a.ncb), dim3(256), 0, st, a); break;
      X(1) X(2) X(4) X(8) X(10) X(12) X(16)
#undef X
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  NE_DISPATCH(a.C, k_ln_mix, dim3(a.R, a.ncb), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ============================================================== copies / fills
__global__ void k_copy_f32(float* d, const float* s, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) d[i] = s[i];
}
__global__ void k_fill_f32(float* d, float v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) d[i] = v;
}

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dst, src, n);
  return hipGetLastError();
}
hipError_t launch_zero_f32(float* dst, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dst, 0.0f, n);
  return hipGetLastError();
}
hipError_t launch_fill_vec(float* dst, float v, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dst, v, n);
  return hipGetLastError();
}

// ============================================================== slot reset
__global__ void k_reset(ResetArgs a) {
  const int k = blockIdx.y;
  const int s = a.slot_idx[k];
  if (s < 0 || (int64_t)s >= a.n_slots) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_err(a.err, ERRB_SLOT_RANGE);
    return;
  }
  float* base = a.pool + (int64_t)s * a.slot_stride;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.slot_stride;
       i += (int64_t)gridDim.x * blockDim.x)
    base[i] = 0.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.counters[s] = 0;
}

hipError_t launch_reset(const ResetArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_reset, dim3(256, a.n), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ============================================================== packing
__global__ void k_pack_matrix(half_t* dst, int64_t dst_ld, const void* src, int src_f16,
                              int64_t rows, int64_t cols) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, c = i % cols;
    const float v = src_f16 ? (float)((const half_t*)src)[i] : ((const float*)src)[i];
    dst[r * dst_ld + c] = (half_t)v;
  }
}

// dst[c][r] = src[r][c]; 64x64 tiles through LDS.
__global__ void k_pack_transpose(half_t* dst, const void* src, int src_f16, int64_t rows,
                                 int64_t cols) {
  __shared__ float tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += blockDim.x) {
    const int rr = i / 64, cc = i % 64;
    const int64_t r = r0 + rr, c = c0 + cc;
    float v = 0.f;
    if (r < rows && c < cols)
      v = src_f16 ? (float)((const half_t*)src)[r * cols + c] : ((const float*)src)[r * cols + c];
    tile[rr][cc] = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += blockDim.x) {
    const int cc = i / 64, rr = i % 64;
    const int64_t r = r0 + rr, c = c0 + cc;
    if (r < rows && c < cols) dst[c * rows + r] = (half_t)tile[rr][cc];
  }
}

__global__ void k_pack_vec(float* dst, const void* src, int src_f16, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src_f16 ? (float)((const half_t*)src)[i] : ((const float*)src)[i];
}

hipError_t launch_pack_matrix(half_t* dst, int64_t dst_ld, const void* src, int src_f16,
                              int64_t rows, int64_t cols, hipStream_t st) {
  const int64_t n = rows * cols;
  const int64_t blocks = n / 256 + 1;
  hipLaunchKernelGGL(k_pack_matrix, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256),
                     0, st, dst, dst_ld, src, src_f16, rows, cols);
  return hipGetLastError();
}
hipError_t launch_pack_transpose(half_t* dst, const void* src, int src_f16, int64_t rows,
                                 int64_t cols, hipStream_t st) {
  hipLaunchKernelGGL(k_pack_transpose, dim3((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64)),
                     dim3(256), 0, st, dst, src, src_f16, rows, cols);
  return hipGetLastError();
}
hipError_t launch_pack_vec(float* dst, const void* src, int src_f16, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(k_pack_vec, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dst, src,
                     src_f16, n);
  return hipGetLastError();
}

// ============================================================== sparse channel-mix value
// One workgroup of 1024 threads per 32-column slice of the value matrix
// (64-byte row segments).  It compacts the union mask in one pass (ascending
// f, deterministic), then gathers h_f * Wv[f, slice] over the whole active
// list, 4 threads per row segment and 256 rows per pass, with
// h = relu(pre)^2 recomputed in fp32 from the stored pre-activation.  The
// sum over rows is reduced in a fixed order (lane shuffles, then the 16
// waves through LDS), added to the residual, and the new channel-mix shift
// of these columns is committed.  Nothing leaves the workgroup half-summed.
constexpr int CMIX_MAXF = 16384;
constexpr int CMIX_MAXB = 4;
constexpr int CMIX_COLS = 32;
constexpr int CMIX_MAXPER = CMIX_MAXF / 256 / 4;  // mask words per compacting thread

// Ascending list of the set bytes of mask[0..F) into s_idx (threads 0..255
// of a 1024-thread workgroup take part; all threads must call it).  Thread t
// owns mask bytes [t*per, (t+1)*per), per = F/256 (a multiple of 4); bytes
// are 0/1, so a word's popcount is its count.  Returns the count.
RW_DEV int cmix_compact(const unsigned char* mask, int F, unsigned short* s_idx, int* s_wcnt) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int words = F / 1024;
  unsigned int mw[CMIX_MAXPER];
  int mine = 0, incl = 0;
  if (t < 256) {
    const unsigned int* m32 = reinterpret_cast<const unsigned int*>(mask) + t * words;
#pragma unroll
    for (int i = 0; i < CMIX_MAXPER; ++i) {
      mw[i] = i < words ? m32[i] : 0u;
      mine += __popc(mw[i]);
    }
    incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_wcnt[wave] = incl;
  }
  __syncthreads();
  const int total = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
  if (t < 256) {
    int pos = incl - mine;
    for (int w = 0; w < wave; ++w) pos += s_wcnt[w];
#pragma unroll
    for (int i = 0; i < CMIX_MAXPER; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if ((mw[i] >> (8 * k)) & 1u) s_idx[pos++] = (unsigned short)(t * words * 4 + 4 * i + k);
    }
  }
  __syncthreads();
  return total;
}

template <int B>
__global__ __launch_bounds__(1024) void k_cmix_sparse(CmixArgs a) {
  __shared__ unsigned short s_idx[CMIX_MAXF];
  __shared__ int s_wcnt[4];
  __shared__ float s_red[16][B][CMIX_COLS];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;

  const int total = cmix_compact(a.mask, a.F, s_idx, s_wcnt);
  if (a.dbg_idx && blockIdx.x == 0) {
    for (int i = t; i < total; i += 1024) a.dbg_idx[i] = s_idx[i];
    if (t == 0) *a.dbg_cnt = total;
  }

  // ---- gather: lane 16 c + g of wave w -> row group rg = 16 w + g (256 of
  // them), columns 8 c .. 8 c + 7 of the slice (the row groups of a chunk
  // are 16 consecutive lanes, summed by DPP).
  // Workgroups are dealt round-robin to the 8 XCDs; consecutive slices go to
  // the same XCD so the two 64-byte halves of a 128-byte line share an L2.
  const int nsl = a.C / CMIX_COLS;
  const int per_xcd = (nsl + 7) / 8;
  const int slice = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (slice >= nsl) return;
  static_assert(CMIX_COLS == 32, "four 8-column chunks per slice");
  const int rg = wave * 16 + (lane & 15);
  const int c8 = (lane >> 4) * 8;
  const int cb = slice * CMIX_COLS + c8;
  float acc[B][8];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;

  // all of a thread's rows (up to CMIX_UNROLL per pass) are loaded before
  // any is used, so a pass costs one memory round trip
  constexpr int CMIX_UNROLL = 8;
  for (int p0 = rg; p0 < total; p0 += 256 * CMIX_UNROLL) {
    u32x4 w4[CMIX_UNROLL];
    float h4[CMIX_UNROLL][B];
#pragma unroll
    for (int u = 0; u < CMIX_UNROLL; ++u) {
      const int p = p0 + 256 * u;
      w4[u] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int b = 0; b < B; ++b) h4[u][b] = 0.f;
      if (p < total) {
        const int f = s_idx[p];
        w4[u] = ld16(a.Wv + (long)f * a.C + cb);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float z = a.pre[(long)b * a.F + f];
          h4[u][b] = z > 0.f ? z * z : 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < CMIX_UNROLL; ++u) {
      const half8 hv = __builtin_bit_cast(half8, w4[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float wf = (float)hv[e];
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b][e] = fmaf(h4[u][b], wf, acc[b][e]);
      }
    }
  }

  // ---- fixed-order reduction: the 16 row groups of a wave by DPP
  // (lane = 16 * column chunk + group), then the 16 waves through LDS
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = sum16(acc[b][e]);
      if ((lane & 15) == 0) s_red[wave][b][c8 + e] = v;
    }
  __syncthreads();
  if (t < B * CMIX_COLS) {
    const int b = t / CMIX_COLS;
    const int col = slice * CMIX_COLS + t % CMIX_COLS;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) sum += s_red[w][b][t % CMIX_COLS];
    a.x[(long)b * a.C + col] += sum;
    if (a.u_ffn) {
      const int slot = a.slots[b];
      if (slot >= 0 && slot < a.n_slots)
        a.pool[(long)slot * a.slot_stride + a.shift_off + col] = a.u_ffn[(long)b * a.C + col];
    }
  }
}

// x += the value partial sums of the fused key projection.  Each workgroup
// owns FOLD_COLS columns: a thread sums 8 of them over partials rg, rg + R,
// ... (R = 1024 / (FOLD_COLS / 8) row groups), then lanes and waves meet in a
// fixed order, so the result does not depend on timing.  32-column slices read whole 128-byte lines of each partial row
// (8-column slices, with four times the workgroups, measured slower).
// Workgroup 0 also writes the debug active list when asked.
constexpr int FOLD_COLS = 32;
template <int B>
__global__ __launch_bounds__(1024) void k_cmix_fold(CmixFoldArgs a) {
  constexpr int CPT = FOLD_COLS / 8;   // threads per row group
  constexpr int RG = 1024 / CPT;       // row groups
  __shared__ float s_red[16][B][FOLD_COLS];
  __shared__ unsigned short s_idx[CMIX_MAXF];
  __shared__ int s_wcnt[4];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int nsl = a.C / FOLD_COLS;
  const int per_xcd = (nsl + 7) / 8;
  const int slice = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (a.dbg_idx && blockIdx.x == 0) {
    const int total = cmix_compact(a.mask, a.F, s_idx, s_wcnt);
    for (int i = t; i < total; i += 1024) a.dbg_idx[i] = s_idx[i];
    if (t == 0) *a.dbg_cnt = total;
  }
  if (slice >= nsl) return;
  // lane 16 c + g of wave w: row group 16 w + g, columns 8 c .. 8 c + 7
  static_assert(CPT == 4, "four 8-column chunks per slice");
  const int rg = wave * 16 + (lane & 15);
  const int c8 = (lane >> 4) * 8;
  const int cb = slice * FOLD_COLS + c8;
  float acc[B][8];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;
  constexpr int U = 4;
  for (int w0 = rg; w0 < a.nwg; w0 += RG * U) {
    floatx4 v[U][B][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = w0 + RG * u;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float* p = a.part + ((long)w * B + b) * a.C + cb;
        v[u][b][0] = w < a.nwg ? ldf4(p) : floatx4{0.f, 0.f, 0.f, 0.f};
        v[u][b][1] = w < a.nwg ? ldf4(p + 4) : floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[b][e] += v[u][b][0][e];
          acc[b][e + 4] += v[u][b][1][e];
        }
  }
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = sum16(acc[b][e]);
      if ((lane & 15) == 0) s_red[wave][b][c8 + e] = v;
    }
  __syncthreads();
  if (t < B * FOLD_COLS) {
    const int b = t / FOLD_COLS;
    const int col = slice * FOLD_COLS + t % FOLD_COLS;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) sum += s_red[w][b][t % FOLD_COLS];
    a.x[(long)b * a.C + col] += sum;
    if (a.u_ffn) {
      const int slot = a.slots[b];
      if (slot >= 0 && slot < a.n_slots)
        a.pool[(long)slot * a.slot_stride + a.shift_off + col] = a.u_ffn[(long)b * a.C + col];
    }
  }
}

hipError_t launch_cmix_fold(const CmixFoldArgs& a, hipStream_t st) {
  if (a.F > CMIX_MAXF || a.F % 1024 || a.C % FOLD_COLS || a.B < 1 || a.B > 2 || a.nwg < 1)
    return hipErrorInvalidValue;
  const dim3 grid((a.C / FOLD_COLS + 7) / 8 * 8);
  if (a.B == 1)
    hipLaunchKernelGGL(k_cmix_fold<1>, grid, dim3(1024), 0, st, a);
  else
    hipLaunchKernelGGL(k_cmix_fold<2>, grid, dim3(1024), 0, st, a);
  return hipGetLastError();
}

int cmix_sparse_max_b() { return CMIX_MAXB; }
const char* cmix_sparse_kernel_name(int B) {
  (void)B;
  return "k_cmix_sparse";
}

hipError_t launch_cmix_sparse(const CmixArgs& a, hipStream_t st) {
  if (a.F > CMIX_MAXF || a.F % 1024 || a.C % CMIX_COLS || a.B < 1 || a.B > CMIX_MAXB)
    return hipErrorInvalidValue;
  const dim3 grid((a.C / CMIX_COLS + 7) / 8 * 8);
  switch (a.B) {
    case 1: hipLaunchKernelGGL(k_cmix_sparse<1>, grid, dim3(1024), 0, st, a); break;
    case 2: hipLaunchKernelGGL(k_cmix_sparse<2>, grid, dim3(1024), 0, st, a); break;
    case 3: hipLaunchKernelGGL(k_cmix_sparse<3>, grid, dim3(1024), 0, st, a); break;
    case 4: hipLaunchKernelGGL(k_cmix_sparse<4>, grid, dim3(1024), 0, st, a); break;
  }
  return hipGetLastError();
}

// ============================================================== penalised greedy
// Pass 1, grid (B, nblk): penalise with the current occurrences, decay them,
// and reduce each block's slice to (max, lowest index).  Pass 2, grid B:
// reduce the block results, write the id and add 1 to its occurrence.
// Every penalty op is a separately rounded fp32 op (no contraction).
RW_DEV bool better(float v, int i, float bv, int bi) {
  if (v != v) return false;       // NaN never wins
  if (bi == INT_MAX) return true;  // first real value
  return v > bv || (v == bv && i < bi);
}

constexpr int GREEDY_PER_BLOCK = 2048;

// Error bits of row b's slot: outside the pool, or listed by an earlier row.
// Such a row reads and updates no occurrence row (two rows naming one slot
// would otherwise update it from two workgroups at once).
// Every thread of the workgroup must call it (the earlier rows are split over
// the threads; it holds a barrier) and gets the same bits.
RW_DEV uint32_t row_slot_bits(const int* slot_idx, int b, int64_t n_slots) {
  const int slot = slot_idx[b];
  if (slot < 0 || (int64_t)slot >= n_slots) return ERRB_SLOT_RANGE;   // the same in every thread
  int dup = 0;
  for (int j = threadIdx.x; j < b; j += blockDim.x) dup |= slot_idx[j] == slot;
  return __syncthreads_or(dup) ? ERRB_SLOT_DUP : 0u;
}

__global__ __launch_bounds__(256) void k_greedy_part(GreedyArgs a) {
  __shared__ float sv[256];
  __shared__ int si[256];
  const int b = blockIdx.x;
  const int blk = blockIdx.y;
  const int slot = a.slot_idx[b];
  const uint32_t bad = row_slot_bits(a.slot_idx, b, a.n_slots);
  if (bad && blk == 0 && threadIdx.x == 0) set_err(a.err, bad);
  float* occ = bad ? nullptr : a.occ + (int64_t)slot * a.V;
  const float pres = a.presence[b], freq = a.frequency[b], dec = a.decay[b];
  const float* lg = a.logits + (int64_t)b * a.V;
  float bv = 0.f;
  int bi = INT_MAX;
  const int v0 = blk * GREEDY_PER_BLOCK;
  const int v1 = min(a.V, v0 + GREEDY_PER_BLOCK);
  for (int v = v0 + threadIdx.x; v < v1; v += 256) {
    float l = lg[v];
    if (occ) {
      const float o = occ[v];
      if (o > 0.f) l = sub_rn(l, add_rn(mul_rn(freq, o), pres));
      occ[v] = mul_rn(o, dec);
    }
    if (better(l, v, bv, bi)) {
      bv = l;
      bi = v;
    }
  }
  sv[threadIdx.x] = bv;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const float v2 = sv[threadIdx.x + o];
      const int i2 = si[threadIdx.x + o];
      if (i2 != INT_MAX && better(v2, i2, sv[threadIdx.x], si[threadIdx.x])) {
        sv[threadIdx.x] = v2;
        si[threadIdx.x] = i2;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.part_val[b * a.nblk + blk] = sv[0];
    a.part_idx[b * a.nblk + blk] = si[0];
  }
}

__global__ __launch_bounds__(64) void k_greedy_final(GreedyArgs a) {
  const int b = blockIdx.x;
  const uint32_t bad = row_slot_bits(a.slot_idx, b, a.n_slots);
  float bv = 0.f;
  int bi = INT_MAX;
  for (int k = threadIdx.x; k < a.nblk; k += 64) {
    const float v = a.part_val[b * a.nblk + k];
    const int i = a.part_idx[b * a.nblk + k];
    if (i != INT_MAX && better(v, i, bv, bi)) {
      bv = v;
      bi = i;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(bv, o);
    const int i2 = __shfl_xor(bi, o);
    if (i2 != INT_MAX && better(v2, i2, bv, bi)) {
      bv = v2;
      bi = i2;
    }
  }
  if (threadIdx.x == 0) {
    int id = bi;
    if (id == INT_MAX) {
      id = 0;
      set_err(a.err, ERRB_ALL_NAN);
    }
    a.ids[b] = id;
    const int slot = a.slot_idx[b];
    if (!bad) {
      float* o = a.occ + (int64_t)slot * a.V + id;
      *o = add_rn(*o, 1.0f);
    }
  }
}

// ---------------------------------------------------------------- sampling
// Penalised temperature / top-k / top-p sampling (the Albatross article's
// adapter defaults and per-step order: forbidden-token mask, presence /
// frequency penalty, batched sampling).  Every decision is integer
// arithmetic so that the pick is reproducible bit for bit:
//   z = l' / T (fp32, l' as in greedy); candidates: not forbidden, z finite;
//   order: the 48-bit key (ordered bits of z) << 16 | (0xFFFF - index), so
//   z descending then index ascending, every key distinct;
//   weight: floor(smp_exp(z - max z) * 2^31), z - max z in fp64;
//   top-k, top-p and the draw each take the shortest prefix of that order
//   whose count or weight sum reaches a goal (k; ceil(p * S_k); floor(u * S)
//   + 1).  The kept sets are prefixes of the whole order and every goal is at
//   most its set's total, so each search runs over the whole order.
// Three launches per call:
//   k_smp_max, grid (G, B): each workgroup takes a chunk of the row and
//     writes the chunk's largest z; it also clears its share of the row's
//     histogram and totals;
//   k_smp_weights, grid (G, B): the row's max from the G partials; key and
//     weight of every token into the workspace; the chunk's histogram over
//     the key's top 12 bits (count and weight sum, integer atomics in LDS)
//     added into the row's histogram; the occurrence decay;
//   k_smp_select, grid B: each search finds its top-level bin from the row's
//     histogram, gathers that bin's tokens into LDS once (a later search in
//     the same bin reuses them) and resolves the remaining 36 bits in three
//     12-bit levels; then occ[id] += 1.
// Integer sums do not depend on the order of the atomics, so neither does
// the result.
constexpr int SMP_THREADS = 1024;   // k_smp_select
constexpr int SMP_PT = 256;         // k_smp_max, k_smp_weights
constexpr int SMP_BINS = 4096;
constexpr int SMP_LIST = 8192;      // tokens gathered into LDS for the finer levels

// exp(t) for t in [-22, 0] (0 below) by a fixed sequence of fp64 operations,
// none fused: Cody and Waite's reduction t = n ln2 + r with ln2 split into
// ln2_hi (40 fractional bits: n * ln2_hi is exact for |n| <= 32) and ln2_lo,
// then the degree-13 Taylor polynomial of exp(r), |r| <= ln2 / 2, by Horner's
// rule (truncation < 5e-18 relative), scaled by 2^n.  The constants are
// 1/ln2, ln2_hi, ln2 - ln2_hi and 1/k!, each rounded to fp64.
RW_DEV double smp_exp(double t) {
#pragma clang fp contract(off)
  if (!(t >= -22.0)) return 0.0;
  constexpr double inv_ln2 = 0x1.71547652b82fep+0;
  constexpr double ln2_hi = 0x1.62e42fefa4000p-1;
  constexpr double ln2_lo = -0x1.8432a1b0e2634p-43;
  constexpr double c[14] = {1.0, 1.0, 1.0 / 2, 1.0 / 6, 1.0 / 24, 1.0 / 120, 1.0 / 720, 1.0 / 5040,
                            1.0 / 40320, 1.0 / 362880, 1.0 / 3628800, 1.0 / 39916800, 1.0 / 479001600,
                            1.0 / 6227020800.0};
  const double n = rint(t * inv_ln2);
  const double r = (t - n * ln2_hi) - n * ln2_lo;
  double p = c[13];
#pragma unroll
  for (int k = 12; k >= 0; --k) p = c[k] + r * p;
  return ldexp(p, (int)n);
}

RW_DEV uint32_t smp_weight(float z, float mx) {
  const double e = smp_exp((double)z - (double)mx);   // exact operands, one rounding
  return (uint32_t)(e * 2147483648.0);                  // exact scaling; truncation = floor
}

RW_DEV uint32_t smp_order_key(float z) {
  const uint32_t b = __float_as_uint(z);
  return (b >> 31) ? ~b : (b | 0x80000000u);
}

// Penalised, tempered logit; NaN marks a token that is not a candidate.
struct SmpRow {
  float pres, freq, T;
  bool greedy;
  RW_DEV float z(float l, float o, bool forb) const {
    const float lp = o > 0.f ? sub_rn(l, add_rn(mul_rn(freq, o), pres)) : l;
    const float x = greedy ? lp : __fdiv_rn(lp, T);
    return (!isfinite(x) || forb) ? NAN : x;
  }
};

RW_DEV SmpRow smp_row(const SampleArgs& a, int b) {
  SmpRow r;
  r.T = a.temperature[b];
  r.pres = a.presence[b];
  r.freq = a.frequency[b];
  r.greedy = !(r.T > 0.f);
  return r;
}

// z from its order key (the inverse of smp_order_key).
RW_DEV float smp_key_z(uint32_t k) { return __uint_as_float((k >> 31) ? (k & 0x7FFFFFFFu) : ~k); }

// Chunk [v0, v1) of the row for workgroup g of G (starts are multiples of 256).
RW_DEV void smp_chunk(int V, int G, int g, int& v0, int& v1) {
  const int ch = ((V + G - 1) / G + SMP_PT - 1) / SMP_PT * SMP_PT;
  v0 = min(V, g * ch);
  v1 = min(V, v0 + ch);
}

// NV consecutive tokens from v (NV = 4: v and v1 multiples of 4, rows 16-byte
// aligned); past v1 a token reads as NaN (not a candidate).
template <int NV>
RW_DEV void smp_load(const float* lg, const float* occ, const unsigned char* forb, int v, int v1, float (&l)[NV],
                     float (&o)[NV], bool (&f)[NV]) {
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    l[e] = NAN;
    o[e] = 0.f;
    f[e] = false;
  }
  if (v >= v1) return;
  if constexpr (NV == 4) {
    const float4 x = *reinterpret_cast<const float4*>(lg + v);
    l[0] = x.x; l[1] = x.y; l[2] = x.z; l[3] = x.w;
    if (occ) {
      const float4 y = *reinterpret_cast<const float4*>(occ + v);
      o[0] = y.x; o[1] = y.y; o[2] = y.z; o[3] = y.w;
    }
    if (forb) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(forb + v);
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = ((w >> (8 * e)) & 0xFFu) != 0u;
    }
  } else {
    l[0] = lg[v];
    if (occ) o[0] = occ[v];
    if (forb) f[0] = forb[v] != 0;
  }
}

template <int NV>
__global__ __launch_bounds__(SMP_PT) void k_smp_max(SampleArgs a) {
  constexpr int U = NV == 4 ? 4 : 8;
  __shared__ float red[SMP_PT / 64];
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x, G = gridDim.x;
  const int nb = SMP_BINS / G;   // G is a power of two <= 64
  for (int i = t; i < nb; i += SMP_PT) {
    a.hcnt[(int64_t)b * SMP_BINS + g * nb + i] = 0u;
    a.hmass[(int64_t)b * SMP_BINS + g * nb + i] = 0ull;
  }
  if (g == 0 && t == 0) {
    a.rown[b] = 0u;
    a.rowtot[b] = 0ull;
  }
  const bool bad = row_slot_bits(a.slot_idx, b, a.n_slots) != 0u;
  const float* occ = bad ? nullptr : a.occ + (int64_t)a.slot_idx[b] * a.V;
  const float* lg = a.logits + (int64_t)b * a.V;
  const SmpRow row = smp_row(a, b);
  int v0, v1;
  smp_chunk(a.V, G, g, v0, v1);
  float mx = -INFINITY;
  for (int base = v0 + NV * t; base < v1; base += SMP_PT * NV * U) {
    float l[U][NV], o[U][NV];
    bool f[U][NV];
#pragma unroll
    for (int i = 0; i < U; ++i) smp_load<NV>(lg, occ, a.forbidden, base + SMP_PT * NV * i, v1, l[i], o[i], f[i]);
#pragma unroll
    for (int i = 0; i < U; ++i)
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        const float x = row.z(l[i][e], o[i][e], f[i][e]);
        if (x == x) mx = fmaxf(mx, x);
      }
  }
  mx = wave_max(mx);
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  if (t == 0) a.pmax[(int64_t)b * SAMPLE_MAX_G + g] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <int NV>
__global__ __launch_bounds__(SMP_PT) void k_smp_weights(SampleArgs a) {
  constexpr int U = NV == 4 ? 4 : 8;
  __shared__ uint32_t hc[SMP_BINS];
  __shared__ unsigned long long hm[SMP_BINS];
  __shared__ unsigned long long red[2][SMP_PT / 64];
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x, G = gridDim.x;
  for (int i = t; i < SMP_BINS; i += SMP_PT) {
    hc[i] = 0u;
    hm[i] = 0ull;
  }
  float mx = -INFINITY;
  for (int j = 0; j < G; ++j) mx = fmaxf(mx, a.pmax[(int64_t)b * SAMPLE_MAX_G + j]);
  const bool bad = row_slot_bits(a.slot_idx, b, a.n_slots) != 0u;
  float* occ = bad ? nullptr : a.occ + (int64_t)a.slot_idx[b] * a.V;
  const float* lg = a.logits + (int64_t)b * a.V;
  uint32_t* key = a.key + (int64_t)b * a.V;
  const SmpRow row = smp_row(a, b);
  const float dec = a.decay[b];
  int v0, v1;
  smp_chunk(a.V, G, g, v0, v1);
  __syncthreads();
  unsigned long long n = 0, tot = 0;
  for (int base = v0 + NV * t; base < v1; base += SMP_PT * NV * U) {
    float l[U][NV], o[U][NV];
    bool f[U][NV];
#pragma unroll
    for (int i = 0; i < U; ++i) smp_load<NV>(lg, occ, a.forbidden, base + SMP_PT * NV * i, v1, l[i], o[i], f[i]);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int v = base + SMP_PT * NV * i;
      if (v >= v1) continue;
      uint32_t k[NV];
      float od[NV];
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        const float x = row.z(l[i][e], o[i][e], f[i][e]);
        const bool c = x == x;
        const uint32_t w = c ? smp_weight(x, mx) : 0u;
        k[e] = c ? smp_order_key(x) : 0u;
        if (c) {
          atomicAdd(&hc[k[e] >> 20], 1u);   // bits 47..36 of the 48-bit key
          atomicAdd(&hm[k[e] >> 20], (unsigned long long)w);
        }
        n += c;
        tot += w;
        od[e] = mul_rn(o[i][e], dec);
      }
      if constexpr (NV == 4) {
        *reinterpret_cast<u32x4*>(key + v) = u32x4{k[0], k[1], k[2], k[3]};
        if (occ) *reinterpret_cast<float4*>(occ + v) = float4{od[0], od[1], od[2], od[3]};
      } else {
        key[v] = k[0];
        if (occ) occ[v] = od[0];
      }
    }
  }
  // wave sums of the two totals, then one atomic each per workgroup
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    n += __shfl_xor(n, o);
    tot += __shfl_xor(tot, o);
  }
  if ((t & 63) == 0) {
    red[0][t >> 6] = n;
    red[1][t >> 6] = tot;
  }
  __syncthreads();
  for (int i = t; i < SMP_BINS; i += SMP_PT) {
    if (hc[i]) {
      atomicAdd(&a.hcnt[(int64_t)b * SMP_BINS + i], hc[i]);
      atomicAdd(&a.hmass[(int64_t)b * SMP_BINS + i], hm[i]);
    }
  }
  if (t == 0) {
    const unsigned long long cn = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    const unsigned long long ct = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    if (cn) {
      atomicAdd(&a.rown[b], (uint32_t)cn);
      atomicAdd(&a.rowtot[b], ct);
    }
  }
}

constexpr int SMP_SMALL = 64;   // a bin this small is resolved by one wave

struct SampleLds {
  uint32_t cnt[SMP_BINS];
  unsigned long long mass[SMP_BINS];
  unsigned long long lkey[SMP_LIST];   // gathered tokens: 48-bit key and weight
  uint32_t lwt[SMP_LIST];
  unsigned long long skey[SMP_SMALL];
  uint32_t swt[SMP_SMALL];
  int lcount, lrange, lbin, scount;    // the list holds every token with digit >= lrange, or digit == lbin
  unsigned long long wtot[2][SMP_THREADS / 64];
  int sel_digit;
  uint32_t sel_cnt;
  unsigned long long sel_c, sel_m;
  unsigned long long res_key, res_m;
};

// Exclusive prefix sums of two values over the 1024 threads (in thread order).
RW_DEV void smp_exscan2(unsigned long long& x, unsigned long long& y, SampleLds& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long ix = x, iy = y;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long nx = __shfl_up(ix, o), ny = __shfl_up(iy, o);
    if (lane >= o) {
      ix += nx;
      iy += ny;
    }
  }
  if (lane == 63) {
    L.wtot[0][wave] = ix;
    L.wtot[1][wave] = iy;
  }
  __syncthreads();
  unsigned long long bx = 0, by = 0;
  for (int w = 0; w < wave; ++w) {
    bx += L.wtot[0][w];
    by += L.wtot[1][w];
  }
  __syncthreads();
  x = bx + ix - x;
  y = by + iy - y;
}

// One level of a search: thread t owns bins 4095 - 4t down to 4092 - 4t (in
// descending key order); the bin where the running count (or weight sum)
// first reaches `goal` goes to L.sel_*.  above_c / above_m: count and weight
// of the tokens before every bin of this level.
RW_DEV void smp_pick(const unsigned long long (&bc)[4], const unsigned long long (&bm)[4], bool by_mass,
                     unsigned long long goal, unsigned long long above_c, unsigned long long above_m, SampleLds& L) {
  const int t = threadIdx.x;
  unsigned long long sc = bc[0] + bc[1] + bc[2] + bc[3], sm = bm[0] + bm[1] + bm[2] + bm[3];
  smp_exscan2(sc, sm, L);
  unsigned long long rc = above_c + sc, rm = above_m + sm;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const unsigned long long before = by_mass ? rm : rc, here = by_mass ? bm[q] : bc[q];
    if (here && before < goal && before + here >= goal) {
      L.sel_digit = SMP_BINS - 1 - 4 * t - q;
      L.sel_cnt = (uint32_t)bc[q];
      L.sel_c = rc;
      L.sel_m = rm;
    }
    rc += bc[q];
    rm += bm[q];
  }
  __syncthreads();
}

// This thread's four bins of a histogram (see smp_pick).
template <typename C, typename M>
RW_DEV void smp_bins(const C* cnt, const M* mass, unsigned long long (&bc)[4], unsigned long long (&bm)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int d = SMP_BINS - 1 - 4 * threadIdx.x - q;
    bc[q] = cnt[d];
    bm[q] = mass[d];
  }
}

// Append (key, weight) to an LDS array, one atomic per wave for the lanes
// that hit; entries at or past `cap` are dropped (the counts bound them).
RW_DEV void smp_append(bool hit, uint64_t c, uint32_t w, int* count, unsigned long long* keys, uint32_t* wts,
                       int cap) {
  const uint64_t m = __ballot(hit);
  if (!m) return;
  const int lane = threadIdx.x & 63, leader = __ffsll((unsigned long long)m) - 1;
  int at = 0;
  if (lane == leader) at = atomicAdd(count, __popcll(m));
  at = __shfl(at, leader);
  const int j = at + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  if (hit && j < cap) {
    keys[j] = c;
    wts[j] = w;
  }
}

RW_DEV uint64_t smp_key48(uint32_t k, int v) { return ((uint64_t)k << 16) | (uint64_t)(0xFFFF - v); }

// Every candidate of the row whose top-level digit is >= d (range) or == d,
// into the LDS list; then the weights of the listed tokens.
template <int NV>
RW_DEV void smp_gather(const uint32_t* key, int V, float mx, int d, bool range, SampleLds& L) {
  constexpr int U = 8;
  const int t = threadIdx.x;
  for (int base = NV * t; base - NV * t < V; base += SMP_THREADS * NV * U) {
    uint32_t k[U][NV];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int v = base + SMP_THREADS * NV * i;
      if constexpr (NV == 4) {
        const u32x4 x = v < V ? *reinterpret_cast<const u32x4*>(key + v) : u32x4{0u, 0u, 0u, 0u};
        k[i][0] = x[0]; k[i][1] = x[1]; k[i][2] = x[2]; k[i][3] = x[3];
      } else {
        k[i][0] = v < V ? key[v] : 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < U; ++i)
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        const int v = base + SMP_THREADS * NV * i + e;
        const int dg = (int)(k[i][e] >> 20);
        const bool hit = k[i][e] != 0u && (range ? dg >= d : dg == d);
        smp_append(hit, smp_key48(k[i][e], v), 0u, &L.lcount, L.lkey, L.lwt, SMP_LIST);
      }
  }
  __syncthreads();
  const int nl = min(L.lcount, SMP_LIST);
  for (int i = threadIdx.x; i < nl; i += SMP_THREADS) L.lwt[i] = smp_weight(smp_key_z((uint32_t)(L.lkey[i] >> 16)), mx);
}

// The few (<= SMP_SMALL) candidates whose keys share `prefix`'s top `bits`
// bits: gathered, then wave 0 finds the first whose running count (weight
// sum) reaches `goal`.  Returns its key; *pm: the weight sum through it.
RW_DEV uint64_t smp_small(const uint32_t* key, int V, float mx, bool listed, uint64_t prefix, int bits,
                          unsigned long long above_c, unsigned long long above_m, bool by_mass,
                          unsigned long long goal, unsigned long long* pm, SampleLds& L) {
  const int t = threadIdx.x, lane = t & 63;
  const int sh = 48 - bits;
  if (t == 0) L.scount = 0;
  __syncthreads();
  if (listed) {
    const int nl = min(L.lcount, SMP_LIST);
    for (int base = 0; base < nl; base += SMP_THREADS) {
      const int i = base + t;
      const uint64_t c = i < nl ? L.lkey[i] : 0ull;
      const bool hit = i < nl && (c >> sh) == (prefix >> sh);
      smp_append(hit, c, hit ? L.lwt[i] : 0u, &L.scount, L.skey, L.swt, SMP_SMALL);
    }
  } else {
    for (int base = 0; base < V; base += SMP_THREADS) {
      const int v = base + t;
      const uint32_t k = v < V ? key[v] : 0u;
      const uint64_t c = smp_key48(k, v);
      const bool hit = k != 0u && (c >> sh) == (prefix >> sh);
      smp_append(hit, c, hit ? smp_weight(smp_key_z(k), mx) : 0u, &L.scount, L.skey, L.swt, SMP_SMALL);
    }
  }
  __syncthreads();
  if (t < 64) {
    const int n = min(L.scount, SMP_SMALL);
    const uint64_t my = lane < n ? L.skey[lane] : 0ull;
    unsigned long long cc = 0, cm = 0;
    for (int j = 0; j < n; ++j) {
      const uint64_t kj = L.skey[j];
      if (kj >= my) {
        cc += 1;
        cm += L.swt[j];
      }
    }
    const bool q = lane < n && (by_mass ? above_m + cm : above_c + cc) >= goal;
    uint64_t best = q ? my : 0ull;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t x = __shfl_xor(best, o);
      best = x > best ? x : best;
    }
    if (q && my == best) {
      L.res_key = best;
      L.res_m = above_m + cm;
    }
  }
  __syncthreads();
  *pm = L.res_m;
  return L.res_key;
}

// The shortest prefix of the row's order whose count (by_mass false) or
// weight sum reaches goal (1 <= goal <= the row's total).  Returns the 48-bit
// key of its last token; *pm: the prefix's weight sum.
template <int NV>
RW_DEV uint64_t smp_search(const SampleArgs& a, int b, float mx, const unsigned long long (&h0c)[4],
                           const unsigned long long (&h0m)[4], bool by_mass, unsigned long long goal,
                           unsigned long long* pm, SampleLds& L) {
  const int t = threadIdx.x;
  const int V = a.V;
  const uint32_t* key = a.key + (int64_t)b * V;
  smp_pick(h0c, h0m, by_mass, goal, 0, 0, L);
  const int d0 = L.sel_digit;
  uint32_t cnt = L.sel_cnt;
  unsigned long long above_c = L.sel_c, above_m = L.sel_m;
  bool listed = d0 >= L.lrange || d0 == L.lbin;   // the same in every thread
  if (!listed && cnt <= SMP_LIST) {
    const bool range = above_c + cnt <= SMP_LIST;
    __syncthreads();
    if (t == 0) {
      L.lcount = 0;
      L.lrange = range ? d0 : SMP_BINS;
      L.lbin = range ? -1 : d0;
    }
    __syncthreads();
    smp_gather<NV>(key, V, mx, d0, range, L);
    __syncthreads();
    listed = true;
  }
  uint64_t prefix = (uint64_t)d0 << 36;
  for (int level = 1;; ++level) {
    if (cnt <= SMP_SMALL || level == 4)   // all 48 bits fixed: one token
      return smp_small(key, V, mx, listed, prefix, 12 * level, above_c, above_m, by_mass, goal, pm, L);
    const int shift = 36 - 12 * level;
    for (int i = t; i < SMP_BINS; i += SMP_THREADS) {
      L.cnt[i] = 0;
      L.mass[i] = 0;
    }
    __syncthreads();
    if (listed) {
      const int nl = min(L.lcount, SMP_LIST);
      for (int i = t; i < nl; i += SMP_THREADS) {
        const uint64_t c = L.lkey[i];
        if ((c >> (shift + 12)) == (prefix >> (shift + 12))) {
          const int d = (int)((c >> shift) & (SMP_BINS - 1));
          atomicAdd(&L.cnt[d], 1u);
          atomicAdd(&L.mass[d], (unsigned long long)L.lwt[i]);
        }
      }
    } else {
      for (int v = t; v < V; v += SMP_THREADS) {
        const uint32_t k = key[v];
        const uint64_t c = smp_key48(k, v);
        if (k != 0u && (c >> (shift + 12)) == (prefix >> (shift + 12))) {
          const int d = (int)((c >> shift) & (SMP_BINS - 1));
          atomicAdd(&L.cnt[d], 1u);
          atomicAdd(&L.mass[d], (unsigned long long)smp_weight(smp_key_z(k), mx));
        }
      }
    }
    __syncthreads();
    unsigned long long bc[4], bm[4];
    smp_bins(L.cnt, L.mass, bc, bm);
    smp_pick(bc, bm, by_mass, goal, above_c, above_m, L);
    prefix |= (uint64_t)L.sel_digit << shift;
    cnt = L.sel_cnt;
    above_c = L.sel_c;
    above_m = L.sel_m;
    __syncthreads();
  }
}

template <int NV>
__global__ __launch_bounds__(SMP_THREADS) void k_smp_select(SampleArgs a) {
  __shared__ SampleLds L;
  const int b = blockIdx.x, t = threadIdx.x;
  const uint32_t bad = row_slot_bits(a.slot_idx, b, a.n_slots);
  if (bad && t == 0) set_err(a.err, bad);
  if (t == 0) {
    L.lcount = 0;
    L.lrange = SMP_BINS;
    L.lbin = -1;
    L.sel_digit = 0;
    L.sel_cnt = 0;
    L.sel_c = L.sel_m = 0;
    L.res_key = L.res_m = 0;
  }
  const unsigned long long n = a.rown[b], tot = a.rowtot[b];
  // the row's max: the G partials, one per lane of every wave
  float mx = (t & 63) < a.G ? a.pmax[(int64_t)b * SAMPLE_MAX_G + (t & 63)] : -INFINITY;
  mx = wave_max(mx);
  unsigned long long h0c[4], h0m[4];   // this thread's bins of the row's top-level histogram
  smp_bins(a.hcnt + (int64_t)b * SMP_BINS, a.hmass + (int64_t)b * SMP_BINS, h0c, h0m);
  const bool greedy = !(a.temperature[b] > 0.f);
  __syncthreads();
  int id = 0;
  if (n == 0) {
    if (t == 0) set_err(a.err, ERRB_ALL_NAN);
  } else {
    const int k = greedy ? 1 : a.top_k[b];
    unsigned long long S = tot;
    if (k > 0 && (unsigned long long)k < n) smp_search<NV>(a, b, mx, h0c, h0m, false, (unsigned long long)k, &S, L);
    const float p = a.top_p[b];
    if (p < 1.f) {
      const double g = ceil((double)p * (double)S);
      smp_search<NV>(a, b, mx, h0c, h0m, true, g < 1.0 ? 1ull : (unsigned long long)g, &S, L);
    }
    float u = a.uniform[b];
    if (!(u >= 0.f)) u = 0.f;
    if (u >= 1.f) u = 0x1.fffffep-1f;
    const unsigned long long target = (unsigned long long)floor((double)u * (double)S);
    unsigned long long m;
    const uint64_t kb = smp_search<NV>(a, b, mx, h0c, h0m, true, target + 1, &m, L);
    id = 0xFFFF - (int)(kb & 0xFFFF);
    if (kb == 0 || id >= a.V) {   // not reachable when every goal is within its set's total
      id = 0;
      if (t == 0) set_err(a.err, ERRB_ALL_NAN);
    }
  }
  if (t == 0) {
    a.ids[b] = id;
    if (!bad) {
      float* o = a.occ + (int64_t)a.slot_idx[b] * a.V + id;
      *o = add_rn(*o, 1.0f);
    }
  }
}

int sample_groups(int B, int V) {
  int G = 1;
  while (G < SAMPLE_MAX_G && (int64_t)B * G * 2 <= 512 && (int64_t)V >= (int64_t)G * 2 * 1024) G *= 2;
  return G;
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t st) {
  if (a.B < 1 || a.V < 1 || a.V > SAMPLE_MAX_V || a.G < 1 || a.G > SAMPLE_MAX_G || (a.G & (a.G - 1)))
    return hipErrorInvalidValue;
  // 16-byte loads and stores when every row starts 16-byte aligned
  const bool vec = a.V % 4 == 0 && (uintptr_t)a.logits % 16 == 0 && (uintptr_t)a.occ % 16 == 0 &&
                   (uintptr_t)a.key % 16 == 0 && (!a.forbidden || (uintptr_t)a.forbidden % 4 == 0);
  if (vec) {
    hipLaunchKernelGGL(k_smp_max<4>, dim3(a.G, a.B), dim3(SMP_PT), 0, st, a);
    hipLaunchKernelGGL(k_smp_weights<4>, dim3(a.G, a.B), dim3(SMP_PT), 0, st, a);
    hipLaunchKernelGGL(k_smp_select<4>, dim3(a.B), dim3(SMP_THREADS), 0, st, a);
  } else {
    hipLaunchKernelGGL(k_smp_max<1>, dim3(a.G, a.B), dim3(SMP_PT), 0, st, a);
    hipLaunchKernelGGL(k_smp_weights<1>, dim3(a.G, a.B), dim3(SMP_PT), 0, st, a);
    hipLaunchKernelGGL(k_smp_select<1>, dim3(a.B), dim3(SMP_THREADS), 0, st, a);
  }
  return hipGetLastError();
}

int greedy_blocks(int V) { return (V + GREEDY_PER_BLOCK - 1) / GREEDY_PER_BLOCK; }

hipError_t launch_greedy(const GreedyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_greedy_part, dim3(a.B, a.nblk), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_greedy_final, dim3(a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}

// ============================================================== int8 weights
// One wave per row: m = max |w| over the row, s = m / 127 (fp32, correctly
// rounded), code q = rint(w / s) clamped to [-127, 127] (0 when s = 0),
// stored as the byte q + 128, and s.  A one-time packing pass.
__global__ __launch_bounds__(256) void k_quant_rows(const half_t* __restrict__ W, int64_t rows, int K,
                                                    uint8_t* __restrict__ q, float* __restrict__ sc) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;   // a whole wave leaves together; no barrier follows
  const half_t* w = W + row * K;
  float m = 0.0f;
  for (int k = lane; k < K; k += 64) m = fmaxf(m, fabsf((float)w[k]));
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float s = m / 127.0f;
  uint8_t* qr = q + row * K;
  for (int k = lane; k < K; k += 64) {
    float r = 0.0f;
    if (s > 0.0f) r = fminf(fmaxf(rintf((float)w[k] / s), -127.0f), 127.0f);
    qr[k] = (uint8_t)((int)r + 128);
  }
  if (lane == 0) sc[row] = s;
}

hipError_t launch_quant_rows(const half_t* W, int64_t rows, int K, uint8_t* q, float* sc, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_rows, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, W, rows, K, q, sc);
  return hipGetLastError();
}

// ---------------------------------------------------------------- measurement
// Streaming read of a buffer: every 16-byte chunk once, grid-stride, four
// independent loads in flight per thread, non-temporal or plain loads.  It
// writes nothing unless the running XOR hits a value no real buffer produces
// (so the loads cannot be dropped); the measured rate is what a kernel of
// this shape can pull from HBM (or from the MALL on a re-read).
template <bool NT>
__global__ __launch_bounds__(256) void k_read_stream(const u32x4* p, int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = NT ? __builtin_nontemporal_load(p + i) : p[i];
    const u32x4 b = NT ? __builtin_nontemporal_load(p + i + stride) : p[i + stride];
    const u32x4 c = NT ? __builtin_nontemporal_load(p + i + 2 * stride) : p[i + 2 * stride];
    const u32x4 d = NT ? __builtin_nontemporal_load(p + i + 3 * stride) : p[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= NT ? __builtin_nontemporal_load(p + i) : p[i];
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == 0x9E3779B9u && sink) sink[0] = v;
}

hipError_t launch_read_stream(const void* buf, int64_t bytes, bool nt, int grid, hipStream_t st) {
  if (!buf || bytes < 16 || grid < 1) return hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  if (nt)
    hipLaunchKernelGGL(k_read_stream<true>, dim3(grid), dim3(256), 0, st, (const u32x4*)buf, n16, (uint32_t*)nullptr);
  else
    hipLaunchKernelGGL(k_read_stream<false>, dim3(grid), dim3(256), 0, st, (const u32x4*)buf, n16, (uint32_t*)nullptr);
  return hipGetLastError();
}
