// WKV-7 kernels.
//
// The RWKV-Server article (section 2 table) describes decode as an O(1)
// update of a fixed-size state and prefill as an O(n) linear scan.  For one
// head the state S is 64x64 fp32, S[i][j] with i the value channel and j the
// key channel, and one token does
//     S <- S diag(d) + (S a) b^T + v k~^T ,   y = S r
// (a = -kappa_hat, b = kappa_hat * alpha), followed by a per-head GroupNorm,
// the (r . k~ . r_k) v bonus and the gate g.
//
// Decode: one workgroup per (row, head).  The head's low-rank adapter
// outputs (decay, alpha, value gate, gate) are computed in the workgroup from
// the 480-ish adapter activations, the state streams through VGPRs once
// (16 floats per thread, 4 threads per value row), and the gated GroupNorm
// output is written in the activation dtype of the next projection.
//
// Prefill: the same per-(token, head) prologue writes d, a, b, k~, v, g and
// the bonus for every token; a scan kernel then runs the recurrence serially
// over tokens with value rows spread over workgroups (rows are independent
// given the per-token vectors), and a post kernel applies GroupNorm + bonus
// + gate.
#include "launch.h"

constexpr int LIN_MAX = 1024;

struct __attribute__((aligned(16))) HeadVecs {
  float r[64], k[64], v[64], d[64], al[64], vg[64], g[64], a[64], bb[64], kt[64], y[64];
  float bonus;
};

// Adapter outputs + keys for row `b` (a token or a batch row), head `h`.
// Leaves r, d, a, bb, kt, v (after the value residual), g and bonus in LDS.
//
// The adapter outputs of the head's 64 channels are dot products of length
// Dw, Da, Dv, Dg.  Per channel the four ranks are taken as one concatenated
// row of NCHK*4 chunks of 8 (ranks are multiples of 8, so a chunk never
// straddles two adapters); thread t works on channel i = t/4 and chunks
// [q*NCHK, (q+1)*NCHK) with q = t%4, and the four quarters meet by shuffle.
// Every global load is issued before the first barrier, so the chain from
// kernel start to the state update is one memory round trip.
template <int NCHK>
RW_DEV void wkv_prologue(const WkvArgs& a, int b, int h, HeadVecs& hv, float* s_lin) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int C = a.C;
  const int i = t >> 2;
  const int qd = t & 3;
  const int c = h * 64 + i;
  const int e1 = a.Dw, e2 = a.Dw + a.Da, e3 = a.Dw + a.Da + a.Dv;

  // every load unconditional and its address picked by selects, so the
  // NCHK loads issue back to back (layer 0 loads its unused value-gate rows
  // too: they are packed like every layer's, and its gate is not applied)
  // the head's adapter block is packed so that load q of thread t is 16-byte
  // chunk q * 256 + t: every wave instruction reads 1 KB contiguously
  u32x4 wch[NCHK];
  const half_t* adp = a.adp + (long)h * NCHK * 2048 + t * 8;
#pragma unroll
  for (int q = 0; q < NCHK; ++q) wch[q] = ld16(adp + q * 2048);
  // per-channel vectors for wave 0's key step
  float k_k = 0.f, k_a = 0.f, r_k = 0.f, vf = 0.f;
  if (wave == 0) {
    const int cc = h * 64 + lane;
    k_k = a.k_k[cc];
    k_a = a.k_a[cc];
    r_k = a.r_k[cc];
    if (a.layer > 0) vf = a.vfirst[(long)b * C + cc];
  }
  float w0 = 0.f, a0 = 0.f, v0 = 0.f;
  if (qd == 0) {
    w0 = a.w0[c];
    a0 = a.a0[c];
    v0 = a.v0[c];
  }
  for (int j = t; j < a.Lin; j += 256) s_lin[j] = a.lin[(long)b * a.Lin + j];
  if (t < 64) {
    const long base = (long)b * 3 * C + h * 64 + t;
    hv.r[t] = a.rkv[base];
    hv.k[t] = a.rkv[base + C];
    hv.v[t] = a.rkv[base + 2 * C];
  }
  __syncthreads();
  {
    float zw = 0.f, za = 0.f, zv = 0.f, zg = 0.f;
#pragma unroll
    for (int q = 0; q < NCHK; ++q) {
      const int e0 = (qd * NCHK + q) * 8;
      int li;
      if (e0 < e1) li = e0;
      else if (e0 < e2) li = a.off_a + (e0 - e1);
      else if (e0 < e3) li = a.off_v + (e0 - e2);
      else li = a.off_g + (e0 - e3);
      const half8 w8 = __builtin_bit_cast(half8, wch[q]);
      // li is a multiple of 8: two 16-byte LDS reads
      const floatx4 x0 = *reinterpret_cast<const floatx4*>(s_lin + li);
      const floatx4 x1 = *reinterpret_cast<const floatx4*>(s_lin + li + 4);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf((float)w8[e], x0[e], s);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf((float)w8[e + 4], x1[e], s);
      zw += e0 < e1 ? s : 0.f;
      za += (e0 >= e1 && e0 < e2) ? s : 0.f;
      zv += (e0 >= e2 && e0 < e3) ? s : 0.f;
      zg += e0 >= e3 ? s : 0.f;
    }
    // the four quarters of a channel are lanes 4i .. 4i+3: quad sums by DPP
    zw += dpp<0xB1>(zw); zw += dpp<0x4E>(zw);
    za += dpp<0xB1>(za); za += dpp<0x4E>(za);
    zv += dpp<0xB1>(zv); zv += dpp<0x4E>(zv);
    zg += dpp<0xB1>(zg); zg += dpp<0x4E>(zg);
    if (qd == 0) {
      // decay = exp(-exp(-softplus(-z) - 0.5)) = exp(-e^{-1/2} sigmoid(z))
      const float sw = 1.0f / (1.0f + expf(-(w0 + zw)));
      hv.d[i] = expf(-0.60653065971263342f * sw);
      hv.al[i] = 1.0f / (1.0f + expf(-(a0 + za)));
      hv.vg[i] = a.layer > 0 ? 1.0f / (1.0f + expf(-(v0 + zv))) : 0.0f;
      hv.g[i] = zg;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int cc = h * 64 + lane;
    const float k = hv.k[lane];
    const float kap = k * k_k;
    const float nrm = sqrtf(wave_sum(kap * kap));
    const float kh = kap / fmaxf(nrm, 1e-12f);
    const float al = hv.al[lane];
    const float kt = k * (1.0f + (al - 1.0f) * k_a);
    hv.a[lane] = -kh;
    hv.bb[lane] = kh * al;
    hv.kt[lane] = kt;
    float v = hv.v[lane];
    if (a.layer == 0)
      a.vfirst[(long)b * C + cc] = v;
    else
      v = v + (vf - v) * hv.vg[lane];
    hv.v[lane] = v;
    const float bon = wave_sum(hv.r[lane] * kt * r_k);
    if (lane == 0) hv.bonus = bon;
  }
  __syncthreads();
}

// Same result when the adapter outputs were computed for all rows by the
// MFMA projection: `lo` holds [rows][4C] = decay | alpha | value gate | gate.
// Register-light, for many rows per launch.
RW_DEV void wkv_prologue_lean(const WkvArgs& a, int b, int h, HeadVecs& hv) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int C = a.C;
  if (wave == 0) {
    const long base = (long)b * 3 * C + h * 64 + lane;
    const float* lo = a.lo + (long)b * 4 * C + h * 64 + lane;
    const int cc = h * 64 + lane;
    const float r = a.rkv[base];
    const float k = a.rkv[base + C];
    float v = a.rkv[base + 2 * C];
    const float al = lo[C];
    const float kap = k * a.k_k[cc];
    const float nrm = sqrtf(wave_sum(kap * kap));
    const float kh = kap / fmaxf(nrm, 1e-12f);
    const float kt = k * (1.0f + (al - 1.0f) * a.k_a[cc]);
    if (a.layer == 0) {
      a.vfirst[(long)b * C + cc] = v;
    } else {
      const float vf = a.vfirst[(long)b * C + cc];
      v = v + (vf - v) * lo[2 * C];
    }
    hv.r[lane] = r;
    hv.d[lane] = lo[0];
    hv.g[lane] = lo[3 * C];
    hv.a[lane] = -kh;
    hv.bb[lane] = kh * al;
    hv.kt[lane] = kt;
    hv.v[lane] = v;
    const float bon = wave_sum(r * kt * a.r_k[cc]);
    if (lane == 0) hv.bonus = bon;
  }
  __syncthreads();
}

// GroupNorm over the head's 64 readouts + bonus * v, times the gate (wave 0);
// gw, gb: this lane's GroupNorm weight and bias (loaded early by the caller).
// The same for a lane that holds its channel's v and gate itself.
RW_DEV float gn_bonus_gate(float y, float v, float g, float bonus, float gw, float gb) {
  const float mean = wave_sum(y) * (1.0f / 64.0f);
  const float dlt = y - mean;
  const float var = wave_sum(dlt * dlt) * (1.0f / 64.0f);
  float o = dlt / sqrtf(var + 64e-5f) * gw + gb;
  o += bonus * v;
  return o * g;
}
RW_DEV float wkv_epilogue(const HeadVecs& hv, float y, float gw, float gb) {
  const int lane = threadIdx.x & 63;
  return gn_bonus_gate(y, hv.v[lane], hv.g[lane], hv.bonus, gw, gb);
}

// State layout in the workgroup: the head's 64 x 64 state is 1024 float4;
// thread t holds float4 number 256 q + t (q = 0..3), i.e. value rows
// 16 q + t / 16 and key columns 4 (t % 16) .. +3.  Each load or store
// instruction of a wave then covers 1 KB of contiguous memory, and the row
// sums (S a and the readout S r) close over the 16 lanes sharing a row.
template <int NCHK>
__global__ __launch_bounds__(256) void k_wkv_decode(WkvArgs a) {
  __shared__ HeadVecs hv;
  __shared__ __attribute__((aligned(16))) float s_lin[NCHK ? LIN_MAX : 4];
  const int b = blockIdx.x / a.H;
  const int h = blockIdx.x % a.H;
  const int t = threadIdx.x;
  const int slot = a.slots[b];
  const bool ok = slot >= 0 && slot < a.n_slots;
  float* base = ok ? a.pool + (long)slot * a.slot_stride + a.layer_off : nullptr;
  float* S = ok ? base + 2L * a.C + (long)h * 4096 + 4 * t : nullptr;
  // the state does not depend on this token: start its loads first
  floatx4 s[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) s[q] = S ? ldf4_nt(S + 1024 * q) : floatx4{0.f, 0.f, 0.f, 0.f};
  float gw = 0.f, gb = 0.f;
  if (t < 64) {
    gw = a.lnx_w[h * 64 + t];
    gb = a.lnx_b[h * 64 + t];
  }
  // the time-mix shift computed by the fused input projection: loaded now,
  // committed at the end (a store here would wait for every load above)
  const bool commit = a.u_att && ok && t >= 64 && t < 128;
  const float u_new = commit ? a.u_att[(long)b * a.C + h * 64 + (t - 64)] : 0.f;
  if constexpr (NCHK == 0)
    wkv_prologue_lean(a, b, h, hv);
  else
    wkv_prologue<NCHK>(a, b, h, hv, s_lin);

  const int j0 = 4 * (t & 15);
  const floatx4 av = *reinterpret_cast<const floatx4*>(&hv.a[j0]);
  const floatx4 bv = *reinterpret_cast<const floatx4*>(&hv.bb[j0]);
  const floatx4 kv = *reinterpret_cast<const floatx4*>(&hv.kt[j0]);
  const floatx4 dv = *reinterpret_cast<const floatx4*>(&hv.d[j0]);
  const floatx4 rv = *reinterpret_cast<const floatx4*>(&hv.r[j0]);
  float y[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 16 * q + (t >> 4);
    const float sa = sum16(s[q][0] * av[0] + s[q][1] * av[1] + s[q][2] * av[2] + s[q][3] * av[3]);
    const float vi = hv.v[i];
    float yy = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float sn = s[q][c] * dv[c] + sa * bv[c] + vi * kv[c];
      s[q][c] = sn;
      yy = fmaf(sn, rv[c], yy);
    }
    y[q] = yy;
  }
  if (S) {
#pragma unroll
    for (int q = 0; q < 4; ++q) stf4_nt(S + 1024 * q, s[q]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float yy = sum16(y[q]);
    if ((t & 15) == 0) hv.y[16 * q + (t >> 4)] = yy;
  }
  __syncthreads();
  if (t < 64) {
    const float o = wkv_epilogue(hv, hv.y[t], gw, gb);
    const long off = (long)b * a.C + h * 64 + t;
    if (a.yout_f16)
      ((half_t*)a.yout)[off] = (half_t)o;
    else
      ((float*)a.yout)[off] = o;
  }
  if (commit) base[h * 64 + (t - 64)] = u_new;
}

// Adapter outputs of 16 tokens (or batch rows) x 16 channels on the fp16
// matrix cores: D = lin_seg (16 x D) W_seg^T (D x 16), 32 ranks per step;
// lane l supplies lin row l % 16 and weight row l % 16, ranks 8 (l / 16) ..
// +7 of the step, and holds D[4 (l / 16) + i][l % 16] in component i.
template <int D>
RW_DEV floatx4 chunk_adapter(const half_t* lin_row, const half_t* w_row) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k0 = 0; k0 < D; k0 += 32) {
    const half8 x = __builtin_bit_cast(half8, ld16(lin_row + k0));
    const half8 y = __builtin_bit_cast(half8, ld16(w_row + k0));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, acc, 0, 0, 0);
  }
  return acc;
}

// Many rows with precomputed adapter outputs: one wave per (row, head), four
// per workgroup.  Lane l owns channel l of the head for the per-channel
// vectors and float4 number 64 q + l (q = 0..15) of the state: value rows
// 4 q + l / 16, key columns 4 (l % 16) .. +3, so every state load and store
// instruction covers 1 KB of contiguous memory and the row sums close over
// 16 lanes.  No lane idles during the per-channel work.
struct WaveVecs {
  float a[64], bb[64], kt[64], d[64], r[64], v[64], y[64];
};

template <int NW>
__global__ __launch_bounds__(64 * NW) void k_wkv_decode_rows(WkvArgs a) {
  __shared__ __attribute__((aligned(16))) WaveVecs wv[NW];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int item = blockIdx.x * NW + wave;       // (row, head) pair
  const bool live = item < a.B * a.H;
  const int b = live ? item / a.H : 0;
  const int h = live ? item % a.H : 0;
  const int C = a.C;
  const int slot = live ? a.slots[b] : -1;
  const bool ok = slot >= 0 && slot < a.n_slots;
  float* S = ok ? a.pool + (long)slot * a.slot_stride + a.layer_off + 2L * C + (long)h * 4096 + 4 * lane
                : nullptr;
  floatx4 s[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) s[q] = S ? ldf4_nt(S + 256 * q) : floatx4{0.f, 0.f, 0.f, 0.f};

  const int cc = h * 64 + lane;
  const long rb = (long)b * 3 * C + cc;
  const float* lo = a.lo + (long)b * 4 * C + cc;
  const float r = a.rkv[rb], k = a.rkv[rb + C];
  float v = a.rkv[rb + 2 * C];
  const float dk = lo[0], al = lo[C], vg = lo[2 * C], g = lo[3 * C];
  const float k_k = a.k_k[cc], k_a = a.k_a[cc], r_k = a.r_k[cc];
  const float gw = a.lnx_w[cc], gb = a.lnx_b[cc];
  const float vf = a.layer > 0 ? a.vfirst[(long)b * C + cc] : 0.f;

  const float kap = k * k_k;
  const float nrm = sqrtf(wave_sum(kap * kap));
  const float kh = kap / fmaxf(nrm, 1e-12f);
  const float kt = k * (1.0f + (al - 1.0f) * k_a);
  if (a.layer == 0) {
    if (live) a.vfirst[(long)b * C + cc] = v;
  } else {
    v = v + (vf - v) * vg;
  }
  const float bonus = wave_sum(r * kt * r_k);
  WaveVecs& w = wv[wave];
  w.a[lane] = -kh;
  w.bb[lane] = kh * al;
  w.kt[lane] = kt;
  w.d[lane] = dk;
  w.r[lane] = r;
  w.v[lane] = v;
  __syncthreads();

  const int j0 = 4 * (lane & 15);
  const floatx4 av = *reinterpret_cast<const floatx4*>(&w.a[j0]);
  const floatx4 bv = *reinterpret_cast<const floatx4*>(&w.bb[j0]);
  const floatx4 kv = *reinterpret_cast<const floatx4*>(&w.kt[j0]);
  const floatx4 dv = *reinterpret_cast<const floatx4*>(&w.d[j0]);
  const floatx4 rv = *reinterpret_cast<const floatx4*>(&w.r[j0]);
  float y[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const float sa = sum16(s[q][0] * av[0] + s[q][1] * av[1] + s[q][2] * av[2] + s[q][3] * av[3]);
    const float vi = w.v[4 * q + (lane >> 4)];
    float yy = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float sn = s[q][c] * dv[c] + sa * bv[c] + vi * kv[c];
      s[q][c] = sn;
      yy = fmaf(sn, rv[c], yy);
    }
    y[q] = yy;
  }
  if (S) {
#pragma unroll
    for (int q = 0; q < 16; ++q) stf4_nt(S + 256 * q, s[q]);
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const float yy = sum16(y[q]);
    if ((lane & 15) == 0) w.y[4 * q + (lane >> 4)] = yy;
  }
  __syncthreads();
  // GroupNorm over the head's readouts, bonus, gate
  const float yl = w.y[lane];
  const float mean = wave_sum(yl) * (1.0f / 64.0f);
  const float dlt = yl - mean;
  const float var = wave_sum(dlt * dlt) * (1.0f / 64.0f);
  const float o = (dlt / sqrtf(var + 64e-5f) * gw + gb + bonus * v) * g;
  if (live) {
    const long off = (long)b * C + cc;
    if (a.yout_f16)
      ((half_t*)a.yout)[off] = (half_t)o;
    else
      ((float*)a.yout)[off] = o;
  }
}

// Many rows with the adapters' second stage computed here instead of by a
// separate MFMA projection: one workgroup per (head, block of 4 RPW rows).
// Wave w first takes channels 16 w .. 16 w + 15 of all four adapters for the
// block's rows on the fp16 matrix cores (as the chunked prefill does for 16
// tokens; the 16-row tile's rows past the block are padding), from the
// block's activation rows that the workgroup stages in LDS once, and passes
// the outputs through LDS to every wave; then rows w RPW .. w RPW + RPW - 1
// one after another, each as k_wkv_decode_rows does for one (row, head).  The
// ranks are template arguments so every load of the adapter step issues at
// once.
// a compile-time integer as a value (ring slots, unrolled trip counts)
template <int U> struct RingSlot { static constexpr int value = U; };

template <int DW, int DA, int DV, int DG, int RPW>
__global__ __launch_bounds__(256) void k_wkv_decode_ad(WkvArgs a) {
  constexpr int RB = 4 * RPW;
  __shared__ __attribute__((aligned(16))) float ad[4][16][64];   // decay | alpha | value gate | gate
  __shared__ __attribute__((aligned(16))) WaveVecs wv[4];
  const int H = a.H, C = a.C;
  const int h = blockIdx.x % H, b0 = (blockIdx.x / H) * RB;
  // wave-uniform as far as the compiler knows too: slot lookups go to scalar loads
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto state_ptr = [&](int rl) -> float* {
    const int b = b0 + rl;
    const int slot = b < a.B ? a.slots[b] : -1;
    return slot >= 0 && slot < a.n_slots
               ? a.pool + (long)slot * a.slot_stride + a.layer_off + 2L * C + (long)h * 4096 + 4 * lane
               : nullptr;
  };
  // Every adapter operand of the wave is loaded at once; then, when the
  // registers allow, the state of the wave's first row, which does not
  // depend on the adapters and so flies during them.  Loads complete in
  // order, so the adapter products wait for their own operands only.
  constexpr int NW_ = DW / 32, NA = DA / 32, NV = DV / 32, NG = DG / 32;
  constexpr bool EARLY = NW_ + NA + NV + NG <= 16;
  const int r16 = lane & 15, k8 = 8 * (lane >> 4);
  const int ch = h * 64 + 16 * wave + r16;   // weight row of this lane
  float* S = EARLY ? state_ptr(wave * RPW) : nullptr;
  const int cc = h * 64 + lane;
  // per-row vectors r, k, v and the value residual's v_first (row clamped)
  auto load_row = [&](int rl, float& r, float& k, float& v, float& vf) {
    const int bc = min(b0 + rl, a.B - 1);
    const long rb = (long)bc * 3 * C + cc;
    r = a.rkv[rb];
    k = a.rkv[rb + C];
    v = a.rkv[rb + 2 * C];
    vf = a.layer > 0 ? a.vfirst[(long)bc * C + cc] : 0.f;
  };
  float r0, k0, v0r, vf0;
  load_row(wave * RPW, r0, k0, v0r, vf0);
  const float k_k = a.k_k[cc], k_a = a.k_a[cc], r_k = a.r_k[cc];
  const float gw = a.lnx_w[cc], gb = a.lnx_b[cc];
  // The block's RB rows of first-stage activations, which all four waves
  // multiply, are loaded once by the workgroup (first, so the LDS stores wait
  // for them only) and shared through LDS in rows padded by 8 halves; tile
  // rows past the block repeat its rows (their products are never read).
  constexpr int XN = DW + DA + DV + DG, XC = XN / 8, XR = XN + 8, XIT = (RB * XC + 255) / 256;
  __shared__ __attribute__((aligned(16))) half_t xs[RB * XR];
  u32x4 xl[XIT];
  {
    const half_t* lin = reinterpret_cast<const half_t*>(a.lin);
#pragma unroll
    for (int i = 0; i < XIT; ++i) {
      const int e0 = i * 256 + (int)threadIdx.x, e = e0 < RB * XC ? e0 : RB * XC - 1;   // loads unconditional
      const int r = e / XC, k = 8 * (e % XC);
      const int src = k < DW ? k : k < DW + DA ? a.off_a + k - DW : k < DW + DA + DV ? a.off_v + k - DW - DA
                                                                                   : a.off_g + k - DW - DA - DV;
      xl[i] = ld16(lin + (long)min(b0 + r, a.B - 1) * a.Lin + src);
    }
  }
  u32x4 yw[NW_], ya[NA], yv[NV], yg[NG];
#pragma unroll
  for (int k = 0; k < NW_; ++k) yw[k] = ld16(a.w2 + (long)ch * DW + k8 + 32 * k);
#pragma unroll
  for (int k = 0; k < NA; ++k) ya[k] = ld16(a.a2 + (long)ch * DA + k8 + 32 * k);
#pragma unroll
  for (int k = 0; k < NV; ++k) yv[k] = ld16(a.v2 + (long)ch * DV + k8 + 32 * k);
#pragma unroll
  for (int k = 0; k < NG; ++k) yg[k] = ld16(a.g2 + (long)ch * DG + k8 + 32 * k);
  const float w0 = a.w0[ch], a0 = a.a0[ch], v0 = a.v0[ch];
  __builtin_amdgcn_sched_barrier(0);
  // a row without a state (no slot, or past B) reads the pool's first floats
  // and zeroes them: unconditional loads keep the waits exact
  auto load_state = [&](floatx4 (&st)[16], const float* p) {
    const float* src = p ? p : a.pool + 4 * lane;
#pragma unroll
    for (int q = 0; q < 16; ++q) st[q] = ldf4_nt(src + 256 * q);
  };
  floatx4 s[16];
  if constexpr (EARLY) load_state(s, S);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < XIT; ++i) {
    const int e = i * 256 + (int)threadIdx.x;
    if (e < RB * XC) *reinterpret_cast<u32x4*>(xs + (e / XC) * XR + 8 * (e % XC)) = xl[i];
  }
  __syncthreads();
  {
    const half_t* xr = xs + (r16 % RB) * XR + k8;
    auto prod = [&](const half_t* x, const u32x4* y, auto n) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < decltype(n)::value; ++k)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const half8*>(x + 32 * k),
                                                    __builtin_bit_cast(half8, y[k]), acc, 0, 0, 0);
      return acc;
    };
    const floatx4 zw = prod(xr, yw, RingSlot<NW_>{}), za = prod(xr + DW, ya, RingSlot<NA>{}),
                  zv = prod(xr + DW + DA, yv, RingSlot<NV>{}), zg = prod(xr + DW + DA + DV, yg, RingSlot<NG>{});
    // lane holds channel 16 w + r16 of rows 4 (lane / 16) + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * (lane >> 4) + i, col = 16 * wave + r16;
      const float sw = 1.0f / (1.0f + expf(-(zw[i] + w0)));
      ad[0][rr][col] = expf(-0.60653065971263342f * sw);     // decay
      ad[1][rr][col] = 1.0f / (1.0f + expf(-(za[i] + a0)));  // alpha
      ad[2][rr][col] = 1.0f / (1.0f + expf(-(zv[i] + v0)));  // value gate
      ad[3][rr][col] = zg[i];                                // gate
    }
  }
  __syncthreads();
  WaveVecs& w = wv[wave];
  for (int j = 0; j < RPW; ++j) {
    const int rl = wave * RPW + j;
    const int b = b0 + rl;
    const bool live = b < a.B;
    float r = r0, k = k0, v = v0r, vf = vf0;
    if (j > 0) load_row(rl, r, k, v, vf);
    if (j > 0 || !EARLY) {
      S = state_ptr(rl);
      load_state(s, S);
    }
    const float dk = ad[0][rl][lane], al = ad[1][rl][lane], vg = ad[2][rl][lane], g = ad[3][rl][lane];

    const float kap = k * k_k;
    const float nrm = sqrtf(wave_sum(kap * kap));
    const float kh = kap / fmaxf(nrm, 1e-12f);
    const float kt = k * (1.0f + (al - 1.0f) * k_a);
    if (a.layer == 0) {
      if (live) a.vfirst[(long)b * C + cc] = v;
    } else {
      v = v + (vf - v) * vg;
    }
    const float bonus = wave_sum(r * kt * r_k);
    w.a[lane] = -kh;
    w.bb[lane] = kh * al;
    w.kt[lane] = kt;
    w.d[lane] = dk;
    w.r[lane] = r;
    w.v[lane] = v;
    __syncthreads();

    const int j0 = 4 * (lane & 15);
    const floatx4 av = *reinterpret_cast<const floatx4*>(&w.a[j0]);
    const floatx4 bv = *reinterpret_cast<const floatx4*>(&w.bb[j0]);
    const floatx4 kv = *reinterpret_cast<const floatx4*>(&w.kt[j0]);
    const floatx4 dv = *reinterpret_cast<const floatx4*>(&w.d[j0]);
    const floatx4 rv = *reinterpret_cast<const floatx4*>(&w.r[j0]);
    if (!S) {
#pragma unroll
      for (int q = 0; q < 16; ++q) s[q] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    float y[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float sa = sum16(s[q][0] * av[0] + s[q][1] * av[1] + s[q][2] * av[2] + s[q][3] * av[3]);
      const float vi = w.v[4 * q + (lane >> 4)];
      float yy = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float sn = s[q][c] * dv[c] + sa * bv[c] + vi * kv[c];
        s[q][c] = sn;
        yy = fmaf(sn, rv[c], yy);
      }
      y[q] = yy;
    }
    if (S) {
#pragma unroll
      for (int q = 0; q < 16; ++q) stf4_nt(S + 256 * q, s[q]);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float yy = sum16(y[q]);
      if ((lane & 15) == 0) w.y[4 * q + (lane >> 4)] = yy;
    }
    __syncthreads();
    // GroupNorm over the head's readouts, bonus, gate
    const float yl = w.y[lane];
    const float mean = wave_sum(yl) * (1.0f / 64.0f);
    const float dlt = yl - mean;
    const float var = wave_sum(dlt * dlt) * (1.0f / 64.0f);
    const float o = (dlt / sqrtf(var + 64e-5f) * gw + gb + bonus * v) * g;
    if (live) {
      const long off = (long)b * C + cc;
      if (a.yout_f16)
        ((half_t*)a.yout)[off] = (half_t)o;
      else
        ((float*)a.yout)[off] = o;
    }
  }
}

// chunks of 8 per thread: (Dw + Da + Dv + Dg) / 32
#define WKV_NCHK_CASES(X) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) \
  X(13) X(14) X(15) X(16) X(17) X(18) X(19) X(20) X(21) X(22) X(23) X(24) X(25) X(26)   \
  X(27) X(28) X(29) X(30) X(31) X(32)

// The decode / prep prologue's adapter layout: per head h, 16-byte chunk
// q * 256 + t holds chunk e = (t % 4) * NCHK + q (8 halves) of channel
// h * 64 + t / 4's concatenated row w2 | a2 | v2 | g2 (NCHK = sum of ranks / 32).
__global__ void k_pack_wkv_adapters(half_t* dst, const half_t* w2, const half_t* a2, const half_t* v2,
                                    const half_t* g2, int C, int Dw, int Da, int Dv, int Dg) {
  const int nchk = (Dw + Da + Dv + Dg) / 32;
  const long chunk = (long)blockIdx.x * 256 + threadIdx.x;
  if (chunk >= (long)C / 64 * nchk * 256) return;
  const int h = (int)(chunk / (nchk * 256));
  const int q = (int)(chunk / 256 % nchk);
  const int t = (int)(chunk % 256);
  const long c = (long)h * 64 + t / 4;
  const int e0 = ((t % 4) * nchk + q) * 8;
  const int e1 = Dw, e2 = Dw + Da, e3 = Dw + Da + Dv;
  const half_t* src = e0 < e1 ? w2 + c * Dw + e0
                    : e0 < e2 ? a2 + c * Da + (e0 - e1)
                    : e0 < e3 ? v2 + c * Dv + (e0 - e2)
                              : g2 + c * Dg + (e0 - e3);
  *reinterpret_cast<u32x4*>(dst + chunk * 8) = *reinterpret_cast<const u32x4*>(src);
}

hipError_t launch_pack_wkv_adapters(half_t* dst, const half_t* w2, const half_t* a2, const half_t* v2,
                                    const half_t* g2, int C, int Dw, int Da, int Dv, int Dg, hipStream_t st) {
  const int dsum = Dw + Da + Dv + Dg;
  if (dsum % 32 || C % 64 || Dw % 8 || Da % 8 || Dv % 8 || Dg % 8) return hipSuccess;   // layout unused then
  const long chunks = (long)C / 64 * (dsum / 32) * 256;
  hipLaunchKernelGGL(k_pack_wkv_adapters, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, dst, w2, a2, v2,
                     g2, C, Dw, Da, Dv, Dg);
  return hipGetLastError();
}

// 0 selects the variant that reads precomputed adapter outputs
static int wkv_nchk(const WkvArgs& a) {
  if (a.lo) return 0;
  const int dsum = a.Dw + a.Da + a.Dv + a.Dg;
  return dsum % 32 ? -1 : dsum / 32;
}

// Waves per workgroup of the many-row kernel: four or five, whichever puts
// fewer waves on the busiest CU when the workgroups are dealt evenly over
// 256 CUs (2560 (row, head) pairs: 512 workgroups of five, two per CU,
// instead of 640 of four, which leave half the CUs a third).
int wkv_rows_waves(int items) {
  const int w4 = (items + 3) / 4, w5 = (items + 4) / 5;
  return (w5 + 255) / 256 * 5 < (w4 + 255) / 256 * 4 ? 5 : 4;
}

// Adapter ranks (Dw, Da, Dv, Dg) with instantiated matrix-core adapter
// steps (the tiny, 2.9B and 7.2B shapes), and whether a launch can use them:
// fp16 first-stage activations at offsets that keep 16-byte loads aligned.
#define CHUNK_AD_CASES(X) X(32, 32, 32, 64) X(64, 64, 32, 320) X(128, 128, 64, 480)
bool wkv_chunk_adapters_ok(const WkvArgs& a) {
  if (a.off_a % 8 || a.off_v % 8 || a.off_g % 8 || a.Lin % 8) return false;
#define X(w, al, v, g) if (a.Dw == w && a.Da == al && a.Dv == v && a.Dg == g) return true;
  CHUNK_AD_CASES(X)
#undef X
  return false;
}

hipError_t launch_wkv_decode(const WkvArgs& a, hipStream_t st) {
  if (a.Lin > LIN_MAX) return hipErrorInvalidValue;
  if (a.ad_rpw && !a.lo && !a.u_att) {
    // many rows, adapters in the kernel: ad_rpw rows per wave
    if (!wkv_chunk_adapters_ok(a) || (a.ad_rpw != 1 && a.ad_rpw != 2 && a.ad_rpw != 4))
      return hipErrorInvalidValue;
    const int rb = 4 * a.ad_rpw;
    const dim3 grid((unsigned)(((a.B + rb - 1) / rb) * a.H));
#define X(w, al, v, g)                                                                              \
  if (a.Dw == w && a.Da == al && a.Dv == v && a.Dg == g) {                                          \
    if (a.ad_rpw == 1) hipLaunchKernelGGL((k_wkv_decode_ad<w, al, v, g, 1>), grid, dim3(256), 0, st, a); \
    else if (a.ad_rpw == 2) hipLaunchKernelGGL((k_wkv_decode_ad<w, al, v, g, 2>), grid, dim3(256), 0, st, a); \
    else hipLaunchKernelGGL((k_wkv_decode_ad<w, al, v, g, 4>), grid, dim3(256), 0, st, a);         \
    return hipGetLastError();                                                                       \
  }
    CHUNK_AD_CASES(X)
#undef X
    return hipErrorInvalidValue;
  }
  if (a.lo && !a.u_att) {
    const int items = a.B * a.H;
    if (wkv_rows_waves(items) == 5)
      hipLaunchKernelGGL(k_wkv_decode_rows<5>, dim3((items + 4) / 5), dim3(320), 0, st, a);
    else
      hipLaunchKernelGGL(k_wkv_decode_rows<4>, dim3((items + 3) / 4), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  switch (wkv_nchk(a)) {
#define X(n) case n: hipLaunchKernelGGL(k_wkv_decode<n>, dim3(a.B * a.H), dim3(256), 0, st, a); break;
    X(0) WKV_NCHK_CASES(X)
#undef X
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- prefill
template <int NCHK>
__global__ __launch_bounds__(256) void k_wkv_prep(WkvArgs a) {
  __shared__ HeadVecs hv;
  __shared__ __attribute__((aligned(16))) float s_lin[LIN_MAX];
  const int tk = blockIdx.x / a.H;
  const int h = blockIdx.x % a.H;
  if constexpr (NCHK == 0)
    wkv_prologue_lean(a, tk, h, hv);
  else
    wkv_prologue<NCHK>(a, tk, h, hv, s_lin);
  const int t = threadIdx.x;
  if (t < 64) {
    const long off = (long)tk * a.C + h * 64 + t;
    a.q_d[off] = hv.d[t];
    a.q_a[off] = hv.a[t];
    a.q_b[off] = hv.bb[t];
    a.q_kt[off] = hv.kt[t];
    a.q_v[off] = hv.v[t];
    a.q_g[off] = hv.g[t];
  }
  if (t == 0) a.q_bonus[(long)tk * a.H + h] = hv.bonus;
  // the scan reads y off the state before its update: y = S (d*r) + (S a)(b.r) + v (kt.r)
  if (t < 64) {
    const float br = wave_sum(hv.bb[t] * hv.r[t]);
    const float kr = wave_sum(hv.kt[t] * hv.r[t]);
    if (t == 0) {
      a.q_brk[((long)tk * a.H + h) * 2] = br;
      a.q_brk[((long)tk * a.H + h) * 2 + 1] = kr;
    }
  }
}

// Grid: H * 4 workgroups; workgroup (h, qb) owns value rows [16 qb, 16 qb + 16)
// of head h: 4 rows per wave, 16 lanes per row, 4 key columns per lane.
// The per-token vectors do not depend on the state, so they are staged
// through LDS in blocks of SCAN_TB tokens, the next block's global loads in
// flight while the current block runs the recurrence; the serial chain per
// token is then LDS reads and ALU only.
constexpr int SCAN_TB = 16;
struct ScanBlock {
  float4 a[SCAN_TB][16], b[SCAN_TB][16], d[SCAN_TB][16], kt[SCAN_TB][16], r[SCAN_TB][16];
  float v[SCAN_TB][16];
  float brk[SCAN_TB][2];   // b.r, kt.r
};

__global__ __launch_bounds__(256) void k_wkv_scan(WkvArgs a) {
  __shared__ ScanBlock sb[2];
  const int h = blockIdx.x >> 2;
  const int qb = blockIdx.x & 3;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int il = wave * 4 + (lane >> 4);    // row inside the workgroup's 16
  const int i = qb * 16 + il;
  const int jq = lane & 15;                 // float4 column index
  const int C = a.C;
  float* S = a.pool + (long)a.seq_slot * a.slot_stride + a.layer_off + 2L * C + (long)h * 4096 +
             i * 64 + 4 * jq;
  float4 s = *reinterpret_cast<const float4*>(S);
  const long cj = h * 64;
  const int T = a.B;

  // staging: 5 vectors x SCAN_TB tokens x 16 float4 = 1280 float4 (5 per
  // thread) plus SCAN_TB x 16 value floats (one per thread)
  float4 ra[5];
  float rvv = 0.f, rbk = 0.f;
  auto load = [&](int t0) {
#pragma unroll
    for (int p = 0; p < 5; ++p) {
      const int e = p * 256 + tid;          // [vec][token][float4]
      const int vec = e / (SCAN_TB * 16);
      const int tk = t0 + (e / 16) % SCAN_TB;
      const int c4 = e % 16;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (tk < T) {
        const long o = (long)tk * C + cj + 4 * c4;
        const float* src = vec == 0 ? a.q_a + o : vec == 1 ? a.q_b + o : vec == 2 ? a.q_d + o
                           : vec == 3 ? a.q_kt + o : a.rkv + (long)tk * 3 * C + cj + 4 * c4;
        x = *reinterpret_cast<const float4*>(src);
      }
      ra[p] = x;
    }
    const int tk = t0 + tid / 16;
    rvv = tk < T ? a.q_v[(long)tk * C + cj + qb * 16 + (tid & 15)] : 0.f;
    const int tb = t0 + (tid >> 1);
    rbk = (tid < 2 * SCAN_TB && tb < T) ? a.q_brk[((long)tb * a.H + h) * 2 + (tid & 1)] : 0.f;
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 5; ++p) {
      const int e = p * 256 + tid;
      const int vec = e / (SCAN_TB * 16);
      const int tt = (e / 16) % SCAN_TB;
      const int c4 = e % 16;
      float4* dst = vec == 0 ? &sb[buf].a[tt][c4] : vec == 1 ? &sb[buf].b[tt][c4]
                    : vec == 2 ? &sb[buf].d[tt][c4] : vec == 3 ? &sb[buf].kt[tt][c4] : &sb[buf].r[tt][c4];
      *dst = ra[p];
    }
    sb[buf].v[tid / 16][tid & 15] = rvv;
    if (tid < 2 * SCAN_TB) sb[buf].brk[tid >> 1][tid & 1] = rbk;
  };

  load(0);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int t0 = 0; t0 < T; t0 += SCAN_TB) {
    const bool more = t0 + SCAN_TB < T;
    if (more) load(t0 + SCAN_TB);
    const ScanBlock& B = sb[buf];
    const int n = T - t0 < SCAN_TB ? T - t0 : SCAN_TB;
    // one token: both row sums read the state before the update, so they run
    // side by side: y = S (d*r) + (S a)(b.r) + v (kt.r), then
    // S <- S diag(d) + (S a) b^T + v kt^T
    auto token = [&](int tt) {
      const float4 av = B.a[tt][jq], bv = B.b[tt][jq], dv = B.d[tt][jq], kv = B.kt[tt][jq];
      const float4 rv = B.r[tt][jq];
      const float vi = B.v[tt][il];
      const float br = B.brk[tt][0], kr = B.brk[tt][1];
      const float4 dr = make_float4(dv.x * rv.x, dv.y * rv.y, dv.z * rv.z, dv.w * rv.w);
      // pairwise partial dots (depth 3), and the update's terms that do not
      // need S a computed while the row sums are in flight
      const float sa = sum16(fmaf(s.y, av.y, s.x * av.x) + fmaf(s.w, av.w, s.z * av.z));
      const float sd = sum16(fmaf(s.y, dr.y, s.x * dr.x) + fmaf(s.w, dr.w, s.z * dr.z));
      const float4 u = make_float4(fmaf(vi, kv.x, s.x * dv.x), fmaf(vi, kv.y, s.y * dv.y),
                                   fmaf(vi, kv.z, s.z * dv.z), fmaf(vi, kv.w, s.w * dv.w));
      s.x = fmaf(sa, bv.x, u.x);
      s.y = fmaf(sa, bv.y, u.y);
      s.z = fmaf(sa, bv.z, u.z);
      s.w = fmaf(sa, bv.w, u.w);
      return sd + sa * br + vi * kr;   // the same in all 16 lanes of the row
    };
    if (n == SCAN_TB) {
      // whole block unrolled and branch-free, so the next token's LDS reads
      // overlap this one: lane jq of each row keeps token jq's readout and
      // stores it after the block
      float ykeep = 0.f;
#pragma unroll
      for (int tt = 0; tt < SCAN_TB; ++tt) {
        const float y = token(tt);
        ykeep = jq == tt ? y : ykeep;
      }
      a.q_y[(long)(t0 + jq) * C + h * 64 + i] = ykeep;
    } else {
      for (int tt = 0; tt < n; ++tt) {
        const float y = token(tt);
        if (jq == 0) a.q_y[(long)(t0 + tt) * C + h * 64 + i] = y;
      }
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  *reinterpret_cast<float4*>(S) = s;
}

// ---------------------------------------------------------------- chunked prefill scan
// The recurrence above, taken CH = 16 tokens at a time in closed form (the
// product of a chunk's transitions diag(d_t) + a_t b_t^T in WY form).  Per
// key column j let l_t = sum_{s <= t} log d_s and define the decayed vectors
//   abar_t = a_t e^{l_{t-1}}, rbar_t = r_t e^{l_t}, bhat_t = b_t e^{-l_t},
//   khat_t = k_t e^{-l_t},    btil_t = b_t e^{l_L - l_t}, ktil_t = k_t e^{l_L - l_t}
// (t = 1..L, l_0 = 0).  With the 16 x 16 matrices C = abar bhat^T and
// E = abar khat^T below the diagonal, F = rbar bhat^T and H = rbar khat^T on
// and below it,
//   A2 = (I - C)^{-1} abar,  G = (I - C)^{-1} E,  K2 = ktil + G^T btil,
//   Q = rbar + F A2,          Z = F G + H,
// the chunk's readouts (rows t of Y) and the state after it are
//   Y = S Q^T + (Z V)^T,      S' = S diag(e^{l_L}) + (S A2^T) btil + V^T K2
// with S the state entering the chunk and V the chunk's values.  Everything
// but the last line is independent of S, so k_wkv_chunk_prep computes it for
// all (chunk, head) pairs at once; k_wkv_chunk_scan then carries S through
// the chunks, two 16-deep contractions per chunk instead of 16 dependent
// rank-1 steps.  Padding tokens (past T) have d = 1 and zero vectors, so they
// change nothing: their columns of Z and rows of K2 are exactly zero, so
// whatever value they carry is multiplied by zero, and a chunk of padding
// only is the identity (e^{l_L} = 1, every other entry 0).  The chunk count
// is padded to a multiple of 3 (the scan's unroll) with such chunks.
constexpr int CH = 16;
// a compile-time integer as a value (ring slots, unrolled trip counts)
__host__ __device__ inline int chunk_count(int T) { return ((T + CH - 1) / CH + 2) / 3 * 3; }
// per (chunk, head) record, floats:
//   A2 [16][64] | Q [16][64] | btil^T [64][16] | K2^T [64][16] | Z [16][16] | e^{l_L} [64]
enum : int { R_A2 = 0, R_Q = 1024, R_BT = 2048, R_K2T = 3072, R_Z = 4096, R_EL = 4352, REC = 4416 };

// D += A B over a 4-deep slice on the fp32 matrix cores: lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16] and holds D[4 (l / 16) + i][l % 16]
// in component i.
RW_DEV floatx4 mfma4(float x, float y, floatx4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, acc, 0, 0, 0);
}

struct ChunkPrepLds {
  // ab, rb, bh, kh first hold the adapter outputs (decay, alpha, value gate,
  // gate) when the kernel computes them itself; they are read before the
  // barrier that precedes the first write of the decayed vectors
  float ab[CH][64], rb[CH][64], bh[CH][64], kh[CH][64], bt[CH][64], kt[CH][64], ld[CH][64];
  float a2[CH][64];
  float m[4][CH][CH + 1];   // C, E, F, H
  float g[CH][CH + 1];
};

// Grid: n_chunks * H workgroups of 256 threads; thread (t, j4) = (tid / 16,
// 4 (tid % 16)) owns token t of the chunk and key columns j4..j4+3.  The
// per-token head vectors are formed here (as in the decode prologue: the key
// normalised per head, the in-context rate folded into k~ and b, the value
// residual), the 16 lanes of a token closing the per-head sums; v, the gate
// and the bonus go to q_v, q_g and q_bonus for the scan and the GroupNorm
// kernel.  The adapter outputs (decay, alpha, value gate, gate) are read from
// lo, or (ranks DW, DA, DV, DG > 0) computed here from the first-stage
// activations (fp16 lin) and the second-stage matrices, wave w taking
// channels 16 w .. 16 w + 15 of all four adapters; the ranks are template
// arguments so every load of that step issues at once.
template <int DW, int DA, int DV, int DG>
__global__ __launch_bounds__(256, 3) void k_wkv_chunk_prep(WkvArgs a) {
  constexpr bool AD = DW > 0;
  __shared__ __attribute__((aligned(16))) ChunkPrepLds L;
  const int H = a.H, C = a.C, T = a.B;
  const int c = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x;
  const int t = tid >> 4, j4 = (tid & 15) * 4;
  const int tk = c * CH + t;
  const bool live = tk < T;
  const int tc = live ? tk : T - 1;   // clamped: every load is issued
  const int cc = h * 64 + j4;
  const long ro = (long)tc * 3 * C + cc, xo = (long)tc * C + cc;
  floatx4 av, bv, kv, dv, rv = ldf4(a.rkv + ro);
  const floatx4 kraw = ldf4(a.rkv + ro + C);
  floatx4 vv = ldf4(a.rkv + ro + 2 * C);
  const floatx4 kk = ldf4(a.k_k + cc), ka = ldf4(a.k_a + cc), rk = ldf4(a.r_k + cc);
  const floatx4 vf = ldf4(a.vfirst + xo);   // layer 0 writes it below instead
  floatx4 al, vg, gg;
  if constexpr (AD) {
    const int lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, k8 = 8 * (lane >> 4);
    const int ch = h * 64 + 16 * w + r16;   // weight row of this lane
    // this wave's second-stage weights, all loaded at once
    constexpr int NW_ = DW / 32, NA = DA / 32, NV = DV / 32, NG = DG / 32;
    u32x4 yw[NW_], ya[NA], yv[NV], yg[NG];
#pragma unroll
    for (int k = 0; k < NW_; ++k) yw[k] = ld16(a.w2 + (long)ch * DW + k8 + 32 * k);
#pragma unroll
    for (int k = 0; k < NA; ++k) ya[k] = ld16(a.a2 + (long)ch * DA + k8 + 32 * k);
#pragma unroll
    for (int k = 0; k < NV; ++k) yv[k] = ld16(a.v2 + (long)ch * DV + k8 + 32 * k);
#pragma unroll
    for (int k = 0; k < NG; ++k) yg[k] = ld16(a.g2 + (long)ch * DG + k8 + 32 * k);
    const float w0 = a.w0[ch], a0 = a.a0[ch], v0 = a.v0[ch];
    // The chunk's 16 rows of first-stage activations, which all four waves
    // multiply, go through LDS once instead of being loaded by every wave:
    // row r holds the ranks w | a | v | g at stride XR halves (the 8-half pad
    // puts the 16 rows' fragment reads on distinct banks).  The tile aliases
    // the front of L, which is first written after the products.
    constexpr int XN = DW + DA + DV + DG, XC = XN / 8, XR = XN + 8;
    constexpr int XIT = (CH * XC + 255) / 256;
    static_assert(CH * XR * 2 <= sizeof(ChunkPrepLds), "activation tile fits the LDS block");
    half_t* xs = reinterpret_cast<half_t*>(&L);
    {
      const half_t* lin = reinterpret_cast<const half_t*>(a.lin);
      u32x4 xv[XIT];
#pragma unroll
      for (int i = 0; i < XIT; ++i) {
        const int e0 = i * 256 + tid, e = e0 < CH * XC ? e0 : CH * XC - 1;   // loads unconditional
        const int r = e / XC, k = 8 * (e % XC);
        const int src = k < DW ? k : k < DW + DA ? a.off_a + k - DW : k < DW + DA + DV ? a.off_v + k - DW - DA
                                                                                     : a.off_g + k - DW - DA - DV;
        const int tr = c * CH + r;
        xv[i] = ld16(lin + (long)(tr < T ? tr : T - 1) * a.Lin + src);
      }
#pragma unroll
      for (int i = 0; i < XIT; ++i) {
        const int e = i * 256 + tid;
        if (e < CH * XC) *reinterpret_cast<u32x4*>(xs + (e / XC) * XR + 8 * (e % XC)) = xv[i];
      }
    }
    __syncthreads();
    const half_t* xr = xs + r16 * XR + k8;
    auto prod = [&](const half_t* x, const u32x4* y, auto n) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < decltype(n)::value; ++k)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const half8*>(x + 32 * k),
                                                    __builtin_bit_cast(half8, y[k]), acc, 0, 0, 0);
      return acc;
    };
    const floatx4 zw = prod(xr, yw, RingSlot<NW_>{});
    const floatx4 za = prod(xr + DW, ya, RingSlot<NA>{});
    const floatx4 zv = prod(xr + DW + DA, yv, RingSlot<NV>{});
    const floatx4 zg = prod(xr + DW + DA + DV, yg, RingSlot<NG>{});
    __syncthreads();   // every wave's fragment reads precede the writes below
    // lane holds channel 16 w + r16 of tokens 4 (lane / 16) + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = 4 * (lane >> 4) + i, col = 16 * w + r16;
      const float sw = 1.0f / (1.0f + expf(-(zw[i] + w0)));
      L.ab[tt][col] = expf(-0.60653065971263342f * sw);     // decay
      L.rb[tt][col] = 1.0f / (1.0f + expf(-(za[i] + a0)));  // alpha
      L.bh[tt][col] = 1.0f / (1.0f + expf(-(zv[i] + v0)));  // value gate
      L.kh[tt][col] = zg[i];                                // gate
    }
    __syncthreads();
    dv = ldf4(&L.ab[t][j4]);
    al = ldf4(&L.rb[t][j4]);
    vg = ldf4(&L.bh[t][j4]);
    gg = ldf4(&L.kh[t][j4]);
  } else {
    const long lo = (long)tc * 4 * C + cc;
    dv = ldf4(a.lo + lo);
    al = ldf4(a.lo + lo + C);
    vg = ldf4(a.lo + lo + 2 * C);
    gg = ldf4(a.lo + lo + 3 * C);
  }
  {
    const floatx4 kap = kraw * kk;
    const float nrm = sqrtf(sum16(kap[0] * kap[0] + kap[1] * kap[1] + kap[2] * kap[2] + kap[3] * kap[3]));
    const float den = fmaxf(nrm, 1e-12f);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float kh = kap[e] / den;
      kv[e] = kraw[e] * (1.0f + (al[e] - 1.0f) * ka[e]);
      av[e] = -kh;
      bv[e] = kh * al[e];
    }
    if (a.layer != 0) vv = vv + (vf - vv) * vg;
    const float bon = sum16(rv[0] * kv[0] * rk[0] + rv[1] * kv[1] * rk[1] + rv[2] * kv[2] * rk[2] +
                            rv[3] * kv[3] * rk[3]);
    if (live) {
      if (a.layer == 0) stf4(a.vfirst + xo, vv);
      stf4(a.q_v + xo, vv);
      stf4(a.q_g + xo, gg);
      if ((tid & 15) == 0) a.q_bonus[(long)tk * H + h] = bon;
    }
  }
  if (!live) {
    av = bv = kv = rv = floatx4{0.f, 0.f, 0.f, 0.f};
    dv = floatx4{1.f, 1.f, 1.f, 1.f};
  }
  floatx4 lg;
#pragma unroll
  for (int e = 0; e < 4; ++e) lg[e] = logf(dv[e]);
  stf4(&L.ld[t][j4], lg);
  __syncthreads();
  // prefix sums of log d: l_{t-1}, l_t and l_L, added in the same order by every thread
  floatx4 run = {0.f, 0.f, 0.f, 0.f}, lm1 = run, lt = run;
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    if (s == t) lm1 = run;
    run += ldf4(&L.ld[s][j4]);
    if (s == t) lt = run;
  }
  floatx4 ab, rb, bh, kh, bt, kt, el;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float em1 = expf(lm1[e]), et = expf(lt[e]), ent = expf(-lt[e]), eLt = expf(run[e] - lt[e]);
    ab[e] = av[e] * em1;
    rb[e] = rv[e] * et;
    bh[e] = bv[e] * ent;
    kh[e] = kv[e] * ent;
    bt[e] = bv[e] * eLt;
    kt[e] = kv[e] * eLt;
    el[e] = expf(run[e]);
  }
  stf4(&L.ab[t][j4], ab);
  stf4(&L.rb[t][j4], rb);
  stf4(&L.bh[t][j4], bh);
  stf4(&L.kh[t][j4], kh);
  stf4(&L.bt[t][j4], bt);
  stf4(&L.kt[t][j4], kt);
  __syncthreads();

  // wave w forms one of C, E, F, H (16 x 16, 64-deep) on the matrix cores;
  // the 64 key columns are visited in 16 slices of 4, lane group g taking
  // columns 16 jb + 4 g + kk of slice 4 jb + kk, so each lane reads float4s
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  {
    const float(*A)[64] = w < 2 ? L.ab : L.rb;
    const float(*B)[64] = (w & 1) ? L.kh : L.bh;
    floatx4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const floatx4 x = ldf4(&A[c16][16 * jb + 4 * g]);
      const floatx4 y = ldf4(&B[c16][16 * jb + 4 * g]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) m = mfma4(x[kk], y[kk], m);
    }
    const bool strict = w < 2;   // C and E exclude the diagonal
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int r = 4 * g + ii;
      L.m[w][r][c16] = (c16 < r || (!strict && c16 == r)) ? m[ii] : 0.f;
    }
  }
  __syncthreads();
  // (I - C) X = [abar | E] by forward substitution, one column per thread
  if (tid < 64 + CH) {
    float x[CH];
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      float v = tid < 64 ? L.ab[r][tid] : L.m[1][r][tid - 64];
#pragma unroll
      for (int s = 0; s < r; ++s) v = fmaf(L.m[0][r][s], x[s], v);
      x[r] = v;
    }
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      if (tid < 64) L.a2[r][tid] = x[r];
      else L.g[r][tid - 64] = x[r];
    }
  }
  __syncthreads();

  float* rec = a.q_rec + ((long)c * H + h) * REC;
  {
    // A2 and Q = rbar + F A2, row t
    const floatx4 a2 = ldf4(&L.a2[t][j4]);
    floatx4 qv = rb;
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      const float f = L.m[2][t][s];
      const floatx4 x = ldf4(&L.a2[s][j4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[e] = fmaf(f, x[e], qv[e]);
    }
    stf4(rec + R_A2 + t * 64 + j4, a2);
    stf4(rec + R_Q + t * 64 + j4, qv);
    if (tid < 16) stf4(rec + R_EL + j4, el);
  }
  {
    // Z = F G + H, entry (t, s)
    const int zt = tid >> 4, zs = tid & 15;
    float z = L.m[3][zt][zs];
#pragma unroll
    for (int u = 0; u < CH; ++u) z = fmaf(L.m[2][zt][u], L.g[u][zs], z);
    rec[R_Z + zt * CH + zs] = z;
  }
  {
    // btil^T and K2^T = ktil^T + btil^T G, key column j, tokens s4..s4+3
    const int j = tid >> 2, s4 = (tid & 3) * 4;
    floatx4 bq, k2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bq[e] = L.bt[s4 + e][j];
      k2[e] = L.kt[s4 + e][j];
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const float bb = L.bt[u][j];
#pragma unroll
      for (int e = 0; e < 4; ++e) k2[e] = fmaf(L.g[u][s4 + e], bb, k2[e]);
    }
    stf4(rec + R_BT + j * CH + s4, bq);
    stf4(rec + R_K2T + j * CH + s4, k2);
  }
}

// Grid: H * 4 workgroups; workgroup (h, q) carries value rows [16 q, 16 q + 16)
// of head h.  Wave w holds the 16 x 16 block of S^T for key columns
// [16 w, 16 w + 16) in the matrix-core accumulator layout (lane l, component
// i: S[16 q + l % 16][16 w + 4 (l / 16) + i]), which is also the operand
// layout of both contractions:
//   readouts  P^T = [A2; Q] S^T   (each wave sums its 16 key columns; the four
//                                  partial tiles meet through LDS)
//   update    S^T <- diag(e^{l_L}) S^T + btil^T (S A2^T)^T + K2^T V
// The chunk records were written just before (too many for L2), so each is
// loaded three chunks ahead into one of three register sets and staged
// through a three-slot LDS ring; the chunk loop is unrolled by three so every
// ring and register index is static, and one barrier per chunk orders the
// ring, the partial sums and the readouts.
struct ChunkBuf {
  float rec[5 * 256 * 4];   // a record (REC floats) in the slots of five float4 per thread
  float vt[16][20];         // V^T of the workgroup's 16 value rows (row stride 20 keeps float4 alignment)
};
struct ChunkRegs {
  floatx4 r[5];
  float v;
};

__global__ __launch_bounds__(256) void k_wkv_chunk_scan(WkvArgs a) {
  __shared__ __attribute__((aligned(16))) ChunkBuf cb[3];
  __shared__ floatx4 xch[3][4][2][64];
  // the four workgroups of a head read the same records: give them one XCD
  // (workgroups are dealt to the eight XCDs round robin) when 8 divides the grid
  const int nwg = 4 * a.H;
  const int lin = nwg % 8 ? (int)blockIdx.x : (blockIdx.x & 7) * (nwg / 8) + (blockIdx.x >> 3);
  const int h = lin >> 2, q = lin & 3;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int C = a.C, T = a.B, H = a.H;
  const int nc = chunk_count(T);
  float* S = a.pool + (long)a.seq_slot * a.slot_stride + a.layer_off + 2L * C + (long)h * 4096 +
             (16 * q + c16) * 64 + 16 * w + 4 * g;
  floatx4 st = ldf4(S);

  // loads are unconditional (chunks past the end repeat the last record and
  // are never read; values past T are clamped to token T - 1 and only meet
  // zeros), so the wait before each staging store is exact
  ChunkRegs rs[3];
  auto load = [&](ChunkRegs& r, int c) {
    c = c < nc ? c : nc - 1;
    const float* rec = a.q_rec + ((long)c * H + h) * REC;
#pragma unroll
    for (int p = 0; p < 5; ++p) {
      const int e = p * 256 + tid;   // slots past the record repeat its last float4
      r.r[p] = ldf4(rec + 4 * (e < REC / 4 ? e : REC / 4 - 1));
    }
    const int tk = c * CH + (tid >> 4);
    r.v = a.q_v[(long)(tk < T ? tk : T - 1) * C + h * 64 + 16 * q + (tid & 15)];
  };
  auto store = [&](const ChunkRegs& r, ChunkBuf& b) {
#pragma unroll
    for (int p = 0; p < 5; ++p) stf4(&b.rec[4 * (p * 256 + tid)], r.r[p]);
    b.vt[tid & 15][tid >> 4] = r.v;
  };

  // chunk c, held in ring slot U = c % 3
  auto chunk = [&](int c, auto slot) {
    constexpr int U = decltype(slot)::value;
    ChunkBuf& B = cb[U];
    // this wave's share of the readout sums: 16 key columns of S A2^T and
    // S Q^T, plus key slice w of Z V; and the update's V^T K2 term, which does
    // not involve S
    floatx4 pa = {0.f, 0.f, 0.f, 0.f}, pq = pa, kv = pa;
    {
      const floatx4 av = ldf4(&B.rec[R_A2 + c16 * 64 + 16 * w + 4 * g]);
      const floatx4 qv = ldf4(&B.rec[R_Q + c16 * 64 + 16 * w + 4 * g]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        pa = mfma4(av[kk], st[kk], pa);
        pq = mfma4(qv[kk], st[kk], pq);
      }
      pq = mfma4(B.rec[R_Z + c16 * CH + 4 * w + g], B.vt[c16][4 * w + g], pq);
      const floatx4 k2 = ldf4(&B.rec[R_K2T + (16 * w + c16) * CH + 4 * g]);
      const floatx4 vq = ldf4(&B.vt[c16][4 * g]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kv = mfma4(k2[kk], vq[kk], kv);
    }
    xch[U][w][0][lane] = pa;
    xch[U][w][1][lane] = pq;
    store(rs[(U + 1) % 3], cb[(U + 1) % 3]);   // chunk c + 1
    __syncthreads();
    load(rs[U], c + 3);
    // the four waves' partial tiles, added in wave order: lane l, component i
    // holds (S A2^T)[16 q + l % 16][4 (l / 16) + i] and likewise the readout
    floatx4 sa = xch[U][0][0][lane], sq = xch[U][0][1][lane];
#pragma unroll
    for (int v = 1; v < 4; ++v) {
      sa += xch[U][v][0][lane];
      sq += xch[U][v][1][lane];
    }
    {
      // wave w stores component w; rows past T land in q_y's padding rows
      const int ty = c * CH + 4 * g + w;
      a.q_y[(long)ty * C + h * 64 + 16 * q + c16] = sq[__builtin_amdgcn_readfirstlane(w)];
    }
    const floatx4 el = ldf4(&B.rec[R_EL + 16 * w + 4 * g]);
    const floatx4 bq = ldf4(&B.rec[R_BT + (16 * w + c16) * CH + 4 * g]);
    st = st * el + kv;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) st = mfma4(bq[kk], sa[kk], st);
  };

  load(rs[0], 0);
  load(rs[1], 1);
  load(rs[2], 2);
  store(rs[0], cb[0]);
  // drain the prologue's loads (issued in an order the loop does not repeat),
  // so the waits inside the loop follow the loop's own order
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  for (int c = 0; c < nc; c += 3) {
    chunk(c, RingSlot<0>{});
    chunk(c + 1, RingSlot<1>{});
    chunk(c + 2, RingSlot<2>{});
  }
  stf4(S, st);
}

// One wave per (token, head), four per workgroup: lane t owns channel t and
// holds its own readout, v and gate, so no LDS and no barrier are needed.
__global__ __launch_bounds__(256) void k_wkv_post(WkvArgs a) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.B * a.H) return;   // whole waves
  const int tk = item / a.H;
  const int h = item % a.H;
  const int t = threadIdx.x & 63;
  const long off = (long)tk * a.C + h * 64 + t;
  const float gw = a.lnx_w[h * 64 + t], gb = a.lnx_b[h * 64 + t];
  const float o = gn_bonus_gate(a.q_y[off], a.q_v[off], a.q_g[off], a.q_bonus[(long)tk * a.H + h], gw, gb);
  if (a.yout_f16)
    ((half_t*)a.yout)[off] = (half_t)o;
  else
    ((float*)a.yout)[off] = o;
}

hipError_t launch_wkv_prep(const WkvArgs& a, hipStream_t st) {
  if (a.Lin > LIN_MAX) return hipErrorInvalidValue;
  switch (wkv_nchk(a)) {
    // precomputed adapters: only wave 0 has work, so one wave per (token, head)
    case 0: hipLaunchKernelGGL(k_wkv_prep<0>, dim3(a.B * a.H), dim3(64), 0, st, a); break;
#define X(n) case n: hipLaunchKernelGGL(k_wkv_prep<n>, dim3(a.B * a.H), dim3(256), 0, st, a); break;
    WKV_NCHK_CASES(X)
#undef X
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
hipError_t launch_wkv_scan(const WkvArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_wkv_scan, dim3(a.H * 4), dim3(256), 0, st, a);
  return hipGetLastError();
}
// adapter ranks (w, a, v, g) with an in-kernel second stage: the tiny, 2.9B and 7.2B shapes
hipError_t launch_wkv_chunk_prep(const WkvArgs& a, hipStream_t st) {
  if (!a.q_rec || a.B < 1) return hipErrorInvalidValue;
  const dim3 grid(chunk_count(a.B) * a.H);
  if (a.lo) {
    hipLaunchKernelGGL((k_wkv_chunk_prep<0, 0, 0, 0>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
#define X(w, al, v, g)                                                                   \
  if (a.Dw == w && a.Da == al && a.Dv == v && a.Dg == g && wkv_chunk_adapters_ok(a)) {   \
    hipLaunchKernelGGL((k_wkv_chunk_prep<w, al, v, g>), grid, dim3(256), 0, st, a);      \
    return hipGetLastError();                                                             \
  }
  CHUNK_AD_CASES(X)
#undef X
  return hipErrorInvalidValue;
}
hipError_t launch_wkv_chunk_scan(const WkvArgs& a, hipStream_t st) {
  if (!a.q_rec || a.B < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_wkv_chunk_scan, dim3(a.H * 4), dim3(256), 0, st, a);
  return hipGetLastError();
}
int64_t wkv_chunk_rec_floats(int T, int H) { return (int64_t)chunk_count(T) * H * REC; }
int wkv_chunk_rows(int T) { return chunk_count(T) * CH; }
hipError_t launch_wkv_post(const WkvArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_wkv_post, dim3((a.B * a.H + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}
