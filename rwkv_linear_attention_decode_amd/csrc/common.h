// Shared device helpers and kernel-argument structs for librwkv7 (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define RW_DEV __device__ __forceinline__

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte loads / stores; the _nt forms are non-temporal (streamed once).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
RW_DEV u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
RW_DEV u32x2 ld8_nt(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)); }
RW_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
RW_DEV u32x4 ld16_nt(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
RW_DEV void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
RW_DEV floatx4 ldf4(const float* p) { return *reinterpret_cast<const floatx4*>(p); }
RW_DEV floatx4 ldf4_nt(const float* p) { return __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p)); }
RW_DEV void stf4(float* p, floatx4 v) { *reinterpret_cast<floatx4*>(p) = v; }
RW_DEV void stf4_nt(float* p, floatx4 v) { __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(p)); }

// device error bits (same values as the public RWKV7_ERR_* macros)
enum : uint32_t {
  ERRB_SLOT_RANGE = 1u,
  ERRB_SLOT_DUP = 2u,
  ERRB_TOKEN_RANGE = 4u,
  ERRB_ALL_NAN = 8u,
};

// epilogues of the projection kernels
enum : int {
  EPI_NONE = 0,      // out_f32 = acc
  EPI_TANH = 1,      // out_f32 = tanh(acc)
  EPI_SIGMOID = 2,   // out_f32 = sigmoid(acc)
  EPI_RESID = 3,     // out_f32 += acc (residual stream)
  EPI_PRE = 4,       // out_f32 = acc + aux[n]; mask[n] = any row > 0
  EPI_RELU2 = 5,     // out_f32 = relu(acc + aux[n])^2
  EPI_DECAY = 6,     // out_f32 = exp(-e^{-1/2} sigmoid(acc + aux[n]))  (WKV decay)
  EPI_SIGB = 7,      // out_f32 = sigmoid(acc + aux[n])
};

// One output block of a fused projection: rows [row0, row1) of the packed
// matrix read activation `act` (row stride ld_act elements) and write
// `out` (row stride ld_out elements) through epilogue `epi`.
struct Seg {
  int row0, row1;
  int epi;
  int ld_act;
  int ld_out;
  int out_f16;       // store the epilogue result as fp16 (the next MFMA projection's input)
  const void* act;
  void* out;
  const float* aux;
  unsigned char* mask;
  const float* mix;  // fused-LayerNorm prologue: token-shift mix of this block
  const half_t* W;   // MFMA path: this block's own matrix [rows][K] (nullptr: the shared one)
  int K;             // ... and its reduction length (a multiple of 32)
  int act_off;       // ... and the column of its activation block inside `act`
};

#define MAX_SEGS 8

enum : int { LNP_NONE = 0, LNP_MIX = 1, LNP_PLAIN = 2 };

// Fused LayerNorm (+ token-shift mix) prologue of the GEMV path: the
// activation of segment s for row b is u + (prev - u) * s.mix with
// u = LN(x[b]) and prev the row's stored shift (LNP_MIX), or u (LNP_PLAIN).
// Workgroup 0 writes u to u_out; a later kernel commits it as the new shift.
struct LnPro {
  const float* x;        // [M][C] residual rows
  const float* g;
  const float* b;
  const float* pool;
  int64_t slot_stride;
  int64_t n_slots;
  int64_t shift_off;
  const int* slots;
  float* u_out;          // [M][C] or nullptr
  int mode;
  int pad_;
};

struct ProjArgs {
  const half_t* W;   // [rows][K] fp16, K contiguous
  int K;
  int M;             // activation rows (batch rows / tokens)
  int nseg;
  int m_tiles;       // MFMA path: number of M tiles
  int split;         // MFMA path: K ranges per tile (1 = the epilogue runs in the GEMM)
  int total_rows;    // MFMA path: output columns over all segments (partial-sum row length)
  float* part;       // MFMA path, split > 1: fp32 partial sums [split][M][total_rows]
  const half_t* vW;  // GEMV key path with the value fused: hidden-major W_val [rows][vC]
  float* vpart;      // ... and its per-workgroup partial sums [workgroups][M][vC]
  int vC;
  // int8 route (GEMV, B <= 2): codes + 128 as bytes [rows][K] and fp32 row
  // scales, used instead of W (and vW) when Wq is set
  const uint8_t* Wq;
  const float* Wsc;
  const uint8_t* vWq;
  const float* vSc;
  int tile0[MAX_SEGS + 1];  // MFMA path: first column tile of each segment (prefix sums)
  LnPro ln;
  Seg seg[MAX_SEGS];
};

RW_DEV float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }


// Sum over each aligned group of 16 lanes, every lane of the group gets the
// same total.  DPP lane moves (VALU): quad_perm [1,0,3,2] and [2,3,0,1],
// then row_half_mirror and row_mirror; each step adds a lane's value to its
// partner's, and partners compute the same commutative sum.
template <int CTRL>
RW_DEV float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
RW_DEV float sum16(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

// Sum over the 64 lanes of a wave (all lanes active): 16-lane sums by DPP,
// then the four row sums read as scalars and added in a fixed order, so
// every lane returns the same value.
RW_DEV float wave_sum(float v) {
  const int s = __builtin_bit_cast(int, sum16(v));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(s, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(s, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(s, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(s, 48));
  return (r0 + r1) + (r2 + r3);
}

RW_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Sum over a 256-thread block; `red` is >= 4 floats of LDS.  All threads get the total.
RW_DEV float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Single fp32 operations rounded to nearest even.  HIP's __fmul_rn
// family are plain operators, which the compiler may fuse into an FMA after
// inlining; these may not be fused.
RW_DEV float mul_rn(float x, float y) {
#pragma clang fp contract(off)
  return x * y;
}
RW_DEV float add_rn(float x, float y) {
#pragma clang fp contract(off)
  return x + y;
}
RW_DEV float sub_rn(float x, float y) {
#pragma clang fp contract(off)
  return x - y;
}

RW_DEV void set_err(uint32_t* err, uint32_t bits) {
  if (err) atomicOr(err, bits);
}

RW_DEV float h2f(half_t h) { return (float)h; }

// Select the segment whose rows contain `row` (segments sorted by row0).
RW_DEV Seg pick_seg(const ProjArgs& a, int row) {
  Seg s = a.seg[0];
#pragma unroll
  for (int i = 1; i < MAX_SEGS; ++i)
    if (i < a.nseg && row >= a.seg[i].row0) s = a.seg[i];
  return s;
}

// The epilogue of segment `s` for a sum v at output column n (relative to
// the segment); `resid` is the stored value EPI_RESID adds to.
RW_DEV float epi_value(const Seg& s, int n, float v, float resid) {
  switch (s.epi) {
    case EPI_TANH: return tanhf(v);
    case EPI_SIGMOID: return sigmoidf_(v);
    case EPI_RESID: return resid + v;
    case EPI_PRE: return v + s.aux[n];
    case EPI_RELU2: {
      const float z = v + s.aux[n];
      return z > 0.0f ? z * z : 0.0f;
    }
    case EPI_DECAY: {
      const float sg = 1.0f / (1.0f + expf(-(v + s.aux[n])));
      return expf(-0.60653065971263342f * sg);
    }
    case EPI_SIGB: return 1.0f / (1.0f + expf(-(v + s.aux[n])));
    default: return v;
  }
}

// Apply the epilogue of segment `s` to output column n (relative to the
// segment), activation row m.
RW_DEV void epi_store(const Seg& s, int n, int m, float v) {
  const long i = (long)m * s.ld_out + n;
  float r;
  switch (s.epi) {
    case EPI_TANH: r = tanhf(v); break;
    case EPI_SIGMOID: r = sigmoidf_(v); break;
    case EPI_RESID: r = (s.out_f16 ? (float)((half_t*)s.out)[i] : ((float*)s.out)[i]) + v; break;
    case EPI_PRE: r = v + s.aux[n]; break;
    case EPI_RELU2: {
      const float z = v + s.aux[n];
      r = z > 0.0f ? z * z : 0.0f;
      break;
    }
    case EPI_DECAY: {
      // exp(-exp(-softplus(-z) - 0.5)) = exp(-e^{-1/2} sigmoid(z))
      const float sg = 1.0f / (1.0f + expf(-(v + s.aux[n])));
      r = expf(-0.60653065971263342f * sg);
      break;
    }
    case EPI_SIGB: r = 1.0f / (1.0f + expf(-(v + s.aux[n]))); break;
    default: r = v; break;
  }
  if (s.out_f16)
    ((half_t*)s.out)[i] = (half_t)r;
  else
    ((float*)s.out)[i] = r;
}
