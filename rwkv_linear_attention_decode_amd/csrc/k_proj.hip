// Projection kernels: fp16 weights [rows][K] (K contiguous) times activations.
//
// The RWKV-Server article (section 3) credits the decode speed of its CUDA
// backend to M=1 specialised linears (a row-1 kernel and a split-K one) and
// switches to dense GEMMs for prefill.  On gfx950 the same split is:
//   * k_gemv  : B <= 4 rows, fp32 activations held in VGPRs, each weight row
//               reduced by one 64-lane (or 32-lane) group with 16-byte
//               non-temporal loads; no split-K partials, so no second pass.
//   * k_gemm  : larger B and prefill, fp16 activations staged in LDS, fp16
//               weights streamed straight from HBM into the B operand of
//               v_mfma_f32_16x16x32_f16 (fp32 accumulate).
#include "launch.h"

#include <stdio.h>

// ============================================================== GEMV
// The fused LayerNorm prologue holds a lane's K slice of every row in VGPRs
// (B * NCH * 8 floats) and the mixed rows in LDS; it is instantiated only
// up to this many floats per lane.
constexpr int kFusedMaxFloats = 80;

// Epilogue family fixed at compile time (GV_MIXED reads it per segment);
// it also gives each projection class its own kernel symbol in traces.
enum : int { GV_MIXED = 0, GV_PRE = 1, GV_RESID = 2, GV_NONE = 3 };

template <int B, int LPR, int NCH, int RPW, int EPK>
__global__ __launch_bounds__(256) void k_gemv(ProjArgs a) {
  constexpr int GPW = 64 / LPR;
  constexpr int ROWS_WAVE = GPW * RPW;
  constexpr int ROWS_WG = 4 * ROWS_WAVE;
  constexpr int K = LPR * NCH * 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane / LPR;
  const int lig = lane % LPR;
  const int row_wg = blockIdx.x * ROWS_WG;
  const Seg sg = pick_seg(a, row_wg);
  const int row_base = row_wg + wave * ROWS_WAVE + grp * RPW;

  u32x4 w[RPW][NCH];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = row_base + i;
    const half_t* wp = a.W + (long)row * K + lig * 8;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (row < sg.row1)
        w[i][c] = ld16_nt(wp + c * LPR * 8);
      else
        w[i][c] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // Activations for this lane's K slice: k = (c * LPR + lig) * 8 + e.
  float xa[B][NCH][8];
  if (a.ln.mode == LNP_NONE) {
    const float* X = reinterpret_cast<const float*>(sg.act);
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const float* xp = X + (long)b * sg.ld_act + (c * LPR + lig) * 8;
        const floatx4 p0 = ldf4(xp), p1 = ldf4(xp + 4);
        xa[b][c][0] = p0.x; xa[b][c][1] = p0.y; xa[b][c][2] = p0.z; xa[b][c][3] = p0.w;
        xa[b][c][4] = p1.x; xa[b][c][5] = p1.y; xa[b][c][6] = p1.z; xa[b][c][7] = p1.w;
      }
  } else if constexpr (B * NCH <= kFusedMaxFloats / 8) {
    // Fused LayerNorm + token-shift mix, computed once per workgroup while
    // the weight loads above are in flight: wave w normalises the quarter
    // [w K/4, (w+1) K/4) of every row (coalesced, stride-64 lanes), row
    // statistics are combined through LDS, and the mixed row is shared
    // through LDS with every wave's K slice.
    constexpr int QK = K / 4;          // elements per wave
    constexpr int PER = QK / 64;       // per lane
    __shared__ __attribute__((aligned(16))) float s_xq[B][K];
    __shared__ float s_st[B][4][2];
    // every global load of the prologue is issued before the first barrier
    float xv[B][PER], gv[PER], bv[PER], mv[PER], pvv[B][PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int k = wave * QK + lane + 64 * j;
      gv[j] = a.ln.g[k];
      bv[j] = a.ln.b[k];
      mv[j] = a.ln.mode == LNP_MIX ? sg.mix[k] : 0.f;
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float* prev = nullptr;
      if (a.ln.mode == LNP_MIX) {
        const int slot = a.ln.slots[b];
        if (slot >= 0 && slot < a.ln.n_slots)
          prev = a.ln.pool + (long)slot * a.ln.slot_stride + a.ln.shift_off;
      }
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int k = wave * QK + lane + 64 * j;
        xv[b][j] = a.ln.x[(long)b * K + k];
        pvv[b][j] = prev ? prev[k] : 0.f;
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float sm = 0.f;
#pragma unroll
      for (int j = 0; j < PER; ++j) sm += xv[b][j];
      sm = wave_sum(sm);
      if (lane == 0) s_st[b][wave][0] = sm;
    }
    __syncthreads();
    float mean[B], rstd[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      mean[b] = (s_st[b][0][0] + s_st[b][1][0] + s_st[b][2][0] + s_st[b][3][0]) * (1.0f / K);
      float q = 0.f;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const float d = xv[b][j] - mean[b];
        q += d * d;
      }
      q = wave_sum(q);
      if (lane == 0) s_st[b][wave][1] = q;
    }
    __syncthreads();
    const bool writer = blockIdx.x == 0 && a.ln.u_out;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      rstd[b] = 1.0f / sqrtf((s_st[b][0][1] + s_st[b][1][1] + s_st[b][2][1] + s_st[b][3][1]) *
                                 (1.0f / K) + 1e-5f);
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int k = wave * QK + lane + 64 * j;
        const float u = (xv[b][j] - mean[b]) * rstd[b] * gv[j] + bv[j];
        if (writer) a.ln.u_out[(long)b * K + k] = u;
        s_xq[b][k] = a.ln.mode == LNP_MIX ? u + (pvv[b][j] - u) * mv[j] : u;
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const float* xp = &s_xq[b][(c * LPR + lig) * 8];
        const floatx4 p0 = *reinterpret_cast<const floatx4*>(xp);
        const floatx4 p1 = *reinterpret_cast<const floatx4*>(xp + 4);
        xa[b][c][0] = p0.x; xa[b][c][1] = p0.y; xa[b][c][2] = p0.z; xa[b][c][3] = p0.w;
        xa[b][c][4] = p1.x; xa[b][c][5] = p1.y; xa[b][c][6] = p1.z; xa[b][c][7] = p1.w;
      }
  }

  float acc[RPW][B];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[i][b] = 0.0f;

#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const half8 h = __builtin_bit_cast(half8, w[i][c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float wf = (float)h[e];
#pragma unroll
        for (int b = 0; b < B; ++b) acc[i][b] = fmaf(wf, xa[b][c][e], acc[i][b]);
      }
    }

#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int o = LPR / 2; o >= 1; o >>= 1) acc[i][b] += __shfl_xor(acc[i][b], o);

  if (lig == 0) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int row = row_base + i;
      if (row < sg.row1) {
        const int n = row - sg.row0;
        const int epi = EPK == GV_PRE ? EPI_PRE : EPK == GV_RESID ? EPI_RESID
                        : EPK == GV_NONE ? EPI_NONE : sg.epi;
        if (epi == EPI_PRE) {
          bool any = false;
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const float pre = acc[i][b] + sg.aux[n];
            ((float*)sg.out)[(long)b * sg.ld_out + n] = pre;
            any |= pre > 0.0f;
          }
          if (sg.mask) sg.mask[n] = any ? 1 : 0;
        } else {
#pragma unroll
          for (int b = 0; b < B; ++b) {
            float* o = (float*)sg.out + (long)b * sg.ld_out + n;
            if (epi == EPI_RESID)
              *o += acc[i][b];
            else if (epi == EPI_NONE)
              *o = acc[i][b];
            else
              epi_store(sg, n, b, acc[i][b]);
          }
        }
      }
    }
  }
}

static constexpr int gemv_rpw(int B) { return B <= 2 ? 4 : 2; }

int gemv_rows_per_wg(int B, int K) {
  const int lpr = (K == 256) ? 32 : 64;
  return 4 * (64 / lpr) * gemv_rpw(B);
}

bool gemv_supported(int B, int K) {
  if (B < 1 || B > 4) return false;
  if (K == 256) return true;
  return K % 512 == 0 && K / 512 >= 1 && K / 512 <= 8;
}

// The fused LayerNorm prologue keeps a lane's whole K slice of every row in
// VGPRs; bound that to 80 floats.
bool gemv_fused_ok(int B, int K) {
  if (!gemv_supported(B, K)) return false;
  const int nch = K == 256 ? 1 : K / 512;
  return B * nch <= kFusedMaxFloats / 8;
}

static int gemv_epk(const ProjArgs& a) {
  int e = a.seg[0].epi;
  for (int i = 1; i < a.nseg; ++i)
    if (a.seg[i].epi != e) return GV_MIXED;
  return e == EPI_PRE ? GV_PRE : e == EPI_RESID ? GV_RESID : e == EPI_NONE ? GV_NONE : GV_MIXED;
}

template <int B, int LPR, int NCH, int RPW>
static void gemv_launch_epk(int epk, dim3 grid, hipStream_t st, const ProjArgs& a) {
  switch (epk) {
    case GV_PRE: hipLaunchKernelGGL((k_gemv<B, LPR, NCH, RPW, GV_PRE>), grid, dim3(256), 0, st, a); break;
    case GV_RESID: hipLaunchKernelGGL((k_gemv<B, LPR, NCH, RPW, GV_RESID>), grid, dim3(256), 0, st, a); break;
    case GV_NONE: hipLaunchKernelGGL((k_gemv<B, LPR, NCH, RPW, GV_NONE>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((k_gemv<B, LPR, NCH, RPW, GV_MIXED>), grid, dim3(256), 0, st, a); break;
  }
}

template <int B>
static hipError_t gemv_dispatch_b(const ProjArgs& a, int total_rows, hipStream_t st) {
  constexpr int RPW = gemv_rpw(B);
  const int K = a.K;
  const int rows_wg = gemv_rows_per_wg(B, K);
  const dim3 grid((total_rows + rows_wg - 1) / rows_wg);
  const int epk = gemv_epk(a);
  if (K == 256) {
    gemv_launch_epk<B, 32, 1, RPW>(epk, grid, st, a);
    return hipGetLastError();
  }
  switch (K / 512) {
#define CASE(n) case n: gemv_launch_epk<B, 64, n, RPW>(epk, grid, st, a); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv(const ProjArgs& a, int total_rows, hipStream_t st) {
  switch (a.M) {
    case 1: return gemv_dispatch_b<1>(a, total_rows, st);
    case 2: return gemv_dispatch_b<2>(a, total_rows, st);
    case 3: return gemv_dispatch_b<3>(a, total_rows, st);
    case 4: return gemv_dispatch_b<4>(a, total_rows, st);
    default: return hipErrorInvalidValue;
  }
}

// Template arguments as a trace prints them, e.g. "k_gemv<1, 64, 5, 4, 1>".
const char* gemv_kernel_name(int B, int K, int epi) {
  static char names[5][9][4][40];
  if (!gemv_supported(B, K)) return "k_gemv";
  const int lpr = K == 256 ? 32 : 64;
  const int nch = K == 256 ? 1 : K / 512;
  const int epk = epi == EPI_PRE ? GV_PRE : epi == EPI_RESID ? GV_RESID
                  : epi == EPI_NONE ? GV_NONE : GV_MIXED;
  char* s = names[B][nch][epk];
  if (!s[0])
    snprintf(s, sizeof(names[0][0][0]), "k_gemv<%d, %d, %d, %d, %d>", B, lpr, nch, gemv_rpw(B), epk);
  return s;
}

// ============================================================== MFMA GEMM
// Workgroup tile: MT activation rows x 64 output columns; 4 waves, each
// owning 16 columns.  K is consumed in chunks of 128: lane l (column l%16,
// group g = l/16) holds 64 contiguous bytes of its weight row, k in
// [32g, 32g+32) of the chunk, used as four 8-wide MFMA K slices.  The A
// operand is read from LDS with the same k mapping, so the product sums
// over every k exactly once.
//
// Activations arrive in fp32 and are split while staged into LDS as
// a = hi + lo * 2^-12 with hi = fp16(a) and lo = fp16((a - hi) * 2^12); each
// weight fragment meets both planes (two MFMAs into two accumulators, the
// second scaled back at the end), so the product keeps ~22 bits of the
// activation while the weights (exact fp16 values) stream once.  The 2^12
// keeps the residual plane out of the fp16 subnormal range.  A single fp16
// rounding of the activations loses too much for deep models whose layers
// amplify relative perturbations.
constexpr float LO_SCALE = 4096.0f;
constexpr float LO_UNSCALE = 1.0f / 4096.0f;
template <int MT>
__global__ __launch_bounds__(256) void k_gemm(ProjArgs a) {
  constexpr int KC = 128;
  constexpr int MT16 = MT / 16;
  constexpr int LDA = KC + 8;  // halves per LDS row (16-byte skew)
  __shared__ __attribute__((aligned(16))) half_t Ah[2][MT][LDA];
  __shared__ __attribute__((aligned(16))) half_t Al[2][MT][LDA];

  // XCD-aware tile order: consecutive tiles (same column tile, successive
  // M tiles) go to the same XCD so its L2 serves the repeated weight reads.
  const int total = a.n_tiles * a.m_tiles;
  const int per_xcd = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int n_tile = lin / a.m_tiles;
  const int m_tile = lin % a.m_tiles;
  const int n0 = n_tile * 64;
  const int m0 = m_tile * MT;
  const Seg sg = pick_seg(a, n0);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int col = n0 + wave * 16 + (lane & 15);
  const bool col_ok = col < sg.row1;
  // a block may carry its own matrix (rows relative to the block) and K
  const bool own = sg.W != nullptr;
  const int K = own ? sg.K : a.K;
  const long wr = own ? (col_ok ? col - sg.row0 : 0) : (col_ok ? col : sg.row0);
  const half_t* wrow = (own ? sg.W : a.W) + wr * K + 32 * g;
  const float* X = reinterpret_cast<const float*>(sg.act) + sg.act_off;
  const int nk = (K + KC - 1) / KC;   // K is a multiple of 32; the last chunk may be partial

  floatx4 acc[MT16], accl[MT16];
#pragma unroll
  for (int t = 0; t < MT16; ++t) {
    acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    accl[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  auto load_w = [&](int kc, u32x4* dst) {
    const half_t* p = wrow + kc * KC;
    const bool ok = kc * KC + 32 * g < K;
#pragma unroll
    for (int s = 0; s < 4; ++s) dst[s] = ok ? ld16_nt(p + 8 * s) : u32x4{0u, 0u, 0u, 0u};
  };
  // MT rows x 128 fp32 = MT*32 float4; 256 threads -> MT/8 float4 each.
  auto load_a = [&](int kc, int buf) {
#pragma unroll
    for (int p = 0; p < MT / 8; ++p) {
      const int idx = p * 256 + threadIdx.x;
      const int r = idx >> 5;
      const int c = (idx & 31) * 4;
      const int m = m0 + r;
      floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
      if (m < a.M && kc * KC + c < K) v = ldf4(X + (long)m * sg.ld_act + kc * KC + c);
      half4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = (half_t)v[e];
        lo[e] = (half_t)((v[e] - (float)hi[e]) * LO_SCALE);
      }
      *reinterpret_cast<half4*>(&Ah[buf][r][c]) = hi;
      *reinterpret_cast<half4*>(&Al[buf][r][c]) = lo;
    }
  };

  u32x4 wf[4], wn[4];
  load_w(0, wf);
  load_a(0, 0);
  __syncthreads();
  int buf = 0;
  for (int kc = 0; kc < nk; ++kc) {
    if (kc + 1 < nk) {
      load_w(kc + 1, wn);
      load_a(kc + 1, buf ^ 1);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const half8 bv = __builtin_bit_cast(half8, wf[s]);
#pragma unroll
      for (int t = 0; t < MT16; ++t) {
        const int r = t * 16 + (lane & 15);
        const int k = 32 * g + 8 * s;
        const half8 ah = *reinterpret_cast<const half8*>(&Ah[buf][r][k]);
        const half8 al = *reinterpret_cast<const half8*>(&Al[buf][r][k]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bv, acc[t], 0, 0, 0);
        accl[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bv, accl[t], 0, 0, 0);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) wf[s] = wn[s];
    buf ^= 1;
  }

  if (!col_ok) return;
  const int n = col - sg.row0;
#pragma unroll
  for (int t = 0; t < MT16; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + t * 16 + 4 * g + i;
      if (m < a.M) {
        const float v = acc[t][i] + accl[t][i] * LO_UNSCALE;
        if (sg.epi == EPI_PRE) {
          ((float*)sg.out)[(long)m * sg.ld_out + n] = v + sg.aux[n];
        } else {
          epi_store(sg, n, m, v);
        }
      }
    }
}

// Union mask of the sparse path when the key projection runs on MFMA:
// computed afterwards from the stored pre-activations.
__global__ void k_pre_mask(const float* pre, int ld, int M, int F, unsigned char* mask) {
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= F) return;
  bool any = false;
  for (int m = 0; m < M; ++m) any |= pre[(long)m * ld + f] > 0.0f;
  mask[f] = any ? 1 : 0;
}

hipError_t launch_gemm(ProjArgs a, int total_rows, hipStream_t st) {
  for (int i = 0; i < a.nseg; ++i) {
    const int K = a.seg[i].W ? a.seg[i].K : a.K;
    if (K % 32 != 0 || K <= 0) return hipErrorInvalidValue;
  }
  a.n_tiles = (total_rows + 63) / 64;
  int mt = a.M <= 16 ? 16 : (a.M <= 32 ? 32 : 64);
  a.m_tiles = (a.M + mt - 1) / mt;
  const int total = a.n_tiles * a.m_tiles;
  const dim3 grid(((total + 7) / 8) * 8);
  if (mt == 16)
    hipLaunchKernelGGL((k_gemm<16>), grid, dim3(256), 0, st, a);
  else if (mt == 32)
    hipLaunchKernelGGL((k_gemm<32>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm<64>), grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int i = 0; i < a.nseg; ++i) {
    const Seg& s = a.seg[i];
    if (s.epi == EPI_PRE && s.mask) {
      const int F = s.row1 - s.row0;
      hipLaunchKernelGGL(k_pre_mask, dim3((F + 255) / 256), dim3(256), 0, st,
                         (const float*)s.out, s.ld_out, a.M, F, s.mask);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

const char* gemm_kernel_name(int M) {
  (void)M;
  return "k_gemm";
}
