// Persistent recurrent sweeps of the fused RNN (gfx950).
//
// Forward: one launch runs every time step of one layer (both directions at
// once) or, for unidirectional stacks, of all layers as a wavefront (layer l
// processes step t while layer l+1 processes step t-1: the "Four layers" row
// of the cuDNN-5 optimisation table in Keras issue #3692).  Each workgroup
// owns U hidden units of one (layer, direction, batch chunk) group, keeps its
// slice of the recurrent weights (and, in the wavefront, of the input weights)
// in registers for the whole sweep -- the persistent-RNN idea discussed in the
// TVM thread "Persist RNN Implementation" -- and per step:
//   1. waits until every producer of the h it needs has published the step
//      (per-workgroup flags, agent scope; GX for the step is prefetched first),
//   2. multiplies the 16-row batch tiles of h_prev by its weight slice on MFMA
//      (K split across the waves, partial tiles summed through LDS in a fixed
//      order),
//   3. applies the cell equations to its units in the same kernel (fused
//      point-wise step of the optimisation table), writes y, the training
//      reserve and the next h into the other half of a ping-pong buffer,
//   4. publishes its flag.
// Backward: the same structure walks time in reverse; each workgroup owns U
// units, exchanges the recurrent gate gradients dG_h, computes
// dh = dG_h W_hh for its units on MFMA, and applies the hand-derived BPTT
// formulas to the reserved forward intermediates.
#include <type_traits>

#include "device_util.h"
#include "rnn_common.h"

using namespace rnnk;

namespace {

template <bool BF16>
using XT = typename std::conditional<BF16, uint16_t, float>::type;

template <bool BF16>
__device__ __forceinline__ XT<BF16> to_x(float v) {
  if constexpr (BF16) return f2bf(v); else return v;
}
template <bool BF16>
__device__ __forceinline__ uint32_t w_bits(const void* base, size_t idx) {
  if constexpr (BF16) return reinterpret_cast<const uint16_t*>(base)[idx];
  else return __float_as_uint(reinterpret_cast<const float*>(base)[idx]);
}
// Pack PER values (bits) into a 16-byte fragment.
template <bool BF16>
__device__ __forceinline__ uint4 pack_frag(const uint32_t (&v)[BF16 ? 8 : 4]) {
  if constexpr (BF16)
    return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
  else
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Wave 0 polls the flags of up to three groups (ranges of nwg workgroups),
// then performs the agent acquire; the workgroup barrier follows.  Returns
// false (for every thread) if the bounded wait expired or another workgroup
// reported an error.
__device__ bool wait_groups(const unsigned* flags, unsigned* err, unsigned spin_limit,
                            const int (&g)[3], int ng, int nwg, unsigned target, int* s_flag) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    const int total = ng * nwg;
    bool ok = false;
    unsigned it = 0;
    while (true) {
      bool mine = true;
#pragma unroll
      for (int i = 0; i < kWaitPerLane; ++i) {
        const int idx = lane + 64 * i;
        if (idx < total) {
          const int gi = idx / nwg;
          const int w = g[gi] * nwg + (idx - gi * nwg);
          mine = mine && (flag_load(flags + (size_t)w * kFlagStride) >= target);
        }
      }
      if (__all(mine)) { ok = true; break; }
      if (++it > spin_limit) { flag_store(err, 1u); break; }
      if ((it & 31u) == 0 && flag_load(err) != 0u) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) *s_flag = ok ? 1 : 0;
    acquire_agent();
  }
  __syncthreads();
  const bool ok = *s_flag != 0;
  __syncthreads();
  return ok;
}

__device__ __forceinline__ void publish(unsigned* flags, unsigned v) {
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    release_agent();
    flag_store(flags + (size_t)blockIdx.x * kFlagStride, v);
  }
}

// ====================================================================== fwd
template <int MODE, bool BF16, int NT, int MT, int KPW, int NW>
__global__ __launch_bounds__(NW * 64) void rnn_fwd_kernel(const FwdParams p) {
  constexpr int G = gates_of(MODE);
  constexpr int R = reserve_slots(MODE);
  constexpr int KC = kchunk<BF16>();
  constexpr int PER = KC / 4;
  constexpr int NCOL = NT * 16;
  constexpr int NROW = MT * 16;
  constexpr int NTHR = NW * 64;
  using X = XT<BF16>;

  __shared__ float red[NW][NROW][NCOL + 1];
  __shared__ float sh_h[NROW * NCOL];
  __shared__ float sh_c[NROW * NCOL];
  __shared__ int s_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fq = lane >> 4;

  const int wg = blockIdx.x;
  const int slice = wg % p.nwg;
  const int grp = wg / p.nwg;
  const int c = grp % p.nchunk;
  const int d = (grp / p.nchunk) % p.D;
  const int li = grp / (p.nchunk * p.D);
  const int layer = p.first_layer + li;
  const int U = p.U, H = p.H, D = p.D, B = p.B, T = p.T, Hp = p.Hp;
  const int GH = G * H;
  const int u0 = slice * U;
  const int Uact = min(U, H - u0);
  const int b0 = c * p.Bc;
  const int Bact = min(p.Bc, B - b0);
  const bool inproj = p.wavefront && li > 0;
  const int GB = (MODE == MODE_GRU && inproj) ? 4 : G;   // column blocks
  const int I_l = p.in_l[li];
  const int Ipx = inproj ? Hp : 0;
  const int nch = (Ipx + Hp) / KC;
  const int DC = p.D * p.nchunk;

  X* xch = reinterpret_cast<X*>(p.xch);
  const size_t gstride = (size_t)2 * p.Bc * Hp;
  X* my_x = xch + (size_t)grp * gstride;
  const X* below_x = inproj ? xch + (size_t)(grp - DC) * gstride : nullptr;
  const void* wih = p.w_ih[li];
  const void* whh = p.w_hh[li];

  // ---- weight slice -> registers (B operand fragments)
  uint4 wf[KPW][NT];
#pragma unroll
  for (int kk = 0; kk < KPW; ++kk) {
    const int gc = wave + kk * NW;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint32_t v[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) v[e] = 0u;
      const int n = nt * 16 + fr;
      const int gb = n / U, j = n - gb * U;
      if (gc < nch && gb < GB && j < Uact) {
        int gate = gb;
        bool use_x = true, use_h = true;
        if (MODE == MODE_GRU && inproj) {
          gate = gb == 3 ? 2 : gb;
          use_x = gb != 3;
          use_h = gb != 2;
        }
        const size_t row = (size_t)d * GH + (size_t)gate * H + u0 + j;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int k = gc * KC + fq * PER + e;
          if (k < Ipx) {
            if (use_x && k < I_l) v[e] = w_bits<BF16>(wih, row * I_l + k);
          } else {
            const int kh = k - Ipx;
            if (use_h && kh < H) v[e] = w_bits<BF16>(whh, row * H + kh);
          }
        }
      }
      wf[kk][nt] = pack_frag<BF16>(v);
    }
  }

  // ---- initial state
  const int q = tid;                   // epilogue pair owned by this thread
  const bool qv = q < Bact * Uact;
  const int qb = qv ? q / Uact : 0, qj = qv ? q - (q / Uact) * Uact : 0;
  const int qu = u0 + qj, qbg = b0 + qb;
  const size_t st_idx = (((size_t)li * D + d) * B + qbg) * H + qu;
  const size_t hx_idx = (((size_t)layer * D + d) * B + qbg) * H + qu;
  if (p.s_begin < 0) {
    if (qv) {
      const float hv = p.h0 ? p.h0[hx_idx] : 0.f;
      const float cv = (MODE == MODE_LSTM && p.c0) ? p.c0[hx_idx] : 0.f;
      sh_h[qb * NCOL + qj] = hv;
      sh_c[qb * NCOL + qj] = cv;
      const int first = p.wavefront ? li : 0;
      my_x[(size_t)(first & 1) * p.Bc * Hp + (size_t)qb * Hp + qu] = to_x<BF16>(hv);
    }
    if (p.persistent) publish(p.flags, 1u);
  } else if (qv) {
    sh_h[qb * NCOL + qj] = p.st_h[st_idx];
    if (MODE == MODE_LSTM) sh_c[qb * NCOL + qj] = p.st_c[st_idx];
  }
  __syncthreads();

  int wgroups[3];
  int nwait = 0;
  if (p.wavefront) {
    for (int o = -1; o <= 1; ++o) {
      const int l2 = li + o;
      if (l2 >= 0 && l2 < p.nlayers) wgroups[nwait++] = grp + o * DC;
    }
  } else {
    wgroups[nwait++] = grp;
  }

  const size_t ystride_t = (size_t)B * D * H;
  for (int s = max(p.s_begin, 0); s < p.s_end; ++s) {
    const int t_rel = p.wavefront ? s - li : s;
    const bool active = t_rel >= 0 && t_rel < T;
    const int t = (d == 0) ? t_rel : T - 1 - t_rel;

    // prefetch the input part of the pre-activations (independent of other workgroups)
    float gxv[4] = {0.f, 0.f, 0.f, 0.f};
    if (active && qv) {
      if (!inproj) {
        const float* g = p.gx + ((size_t)t * B + qbg) * D * GH + (size_t)d * GH + qu;
#pragma unroll
        for (int gi = 0; gi < G; ++gi) gxv[gi] = g[(size_t)gi * H];
      } else {
        const float* bi = p.b_ih[li] + (size_t)d * GH + qu;
        const float* bh = p.b_hh[li] + (size_t)d * GH + qu;
        if (MODE == MODE_GRU) {
          gxv[0] = bi[0] + bh[0];
          gxv[1] = bi[H] + bh[H];
          gxv[2] = bi[2 * H];   // b_in (x part of n)
          gxv[3] = bh[2 * H];   // b_hn (h part of n)
        } else {
#pragma unroll
          for (int gi = 0; gi < G; ++gi) gxv[gi] = bi[(size_t)gi * H] + bh[(size_t)gi * H];
        }
      }
    }
    float bhn = 0.f;
    if (MODE == MODE_GRU && !inproj && active && qv) bhn = p.b_hh[li][(size_t)d * GH + 2 * H + qu];

    if (p.persistent) {
      if (!wait_groups(p.flags, p.err, p.spin_limit, wgroups, nwait, p.nwg, (unsigned)(s + 1), &s_flag))
        return;
    }

    if (active) {
      f32x4 acc[MT][NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const X* hsrc = my_x + (size_t)(s & 1) * p.Bc * Hp;
      const X* xsrc = inproj ? below_x + (size_t)(s & 1) * p.Bc * Hp : nullptr;
#pragma unroll
      for (int kk = 0; kk < KPW; ++kk) {
        const int gc = wave + kk * NW;
        if (gc < nch) {
          const int k0 = gc * KC + fq * PER;
          const X* src = (k0 < Ipx) ? xsrc + k0 : hsrc + (k0 - Ipx);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int row = mt * 16 + fr;
            uint4 a = make_uint4(0u, 0u, 0u, 0u);
            if (row < Bact) a = *reinterpret_cast<const uint4*>(src + (size_t)row * Hp);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma_chunk<BF16>(a, wf[kk][nt], acc[mt][nt]);
          }
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[wave][mt * 16 + fq * 4 + r][nt * 16 + fr] = acc[mt][nt][r];
      __syncthreads();

      if (qv) {
        float pre[4];
#pragma unroll
        for (int gb = 0; gb < 4; ++gb) {
          float v = 0.f;
          if (gb < GB) {
#pragma unroll
            for (int w = 0; w < NW; ++w) v += red[w][qb][gb * U + qj];
          }
          pre[gb] = v;
        }
        const float hprev = sh_h[qb * NCOL + qj];
        float hnew;
        float* res = (p.training && R > 0)
                         ? p.reserve[li] + (((size_t)d * T + t) * B + qbg) * R * H + qu
                         : nullptr;
        if (MODE == MODE_LSTM) {
          const float ig = sigmoidf_(pre[0] + gxv[0]);
          const float fg = sigmoidf_(pre[1] + gxv[1]);
          const float gg = tanhf(pre[2] + gxv[2]);
          const float og = sigmoidf_(pre[3] + gxv[3]);
          const float cn = fg * sh_c[qb * NCOL + qj] + ig * gg;
          hnew = og * tanhf(cn);
          sh_c[qb * NCOL + qj] = cn;
          if (res) {
            res[0] = ig; res[H] = fg; res[2 * H] = gg; res[3 * H] = og; res[4 * H] = cn;
          }
        } else if (MODE == MODE_GRU) {
          const float rg = sigmoidf_(pre[0] + gxv[0]);
          const float zg = sigmoidf_(pre[1] + gxv[1]);
          float ghn, gin;
          if (inproj) { gin = pre[2] + gxv[2]; ghn = pre[3] + gxv[3]; }
          else { gin = gxv[2]; ghn = pre[2] + bhn; }
          const float ng = tanhf(gin + rg * ghn);
          hnew = (1.f - zg) * ng + zg * hprev;
          if (res) { res[0] = rg; res[H] = zg; res[2 * H] = ng; res[3 * H] = ghn; }
        } else {
          hnew = tanhf(pre[0] + gxv[0]);
        }
        sh_h[qb * NCOL + qj] = hnew;
        p.y[li][(size_t)t * ystride_t + (size_t)qbg * D * H + (size_t)d * H + qu] = hnew;
        my_x[(size_t)((s + 1) & 1) * p.Bc * Hp + (size_t)qb * Hp + qu] = to_x<BF16>(hnew);
      }
    }
    if (p.persistent) publish(p.flags, (unsigned)(s + 2));
    __syncthreads();
  }

  if (qv) {
    if (p.s_end >= p.s_total) {
      if (p.hy) p.hy[hx_idx] = sh_h[qb * NCOL + qj];
      if (MODE == MODE_LSTM && p.cy) p.cy[hx_idx] = sh_c[qb * NCOL + qj];
    } else {
      p.st_h[st_idx] = sh_h[qb * NCOL + qj];
      if (MODE == MODE_LSTM) p.st_c[st_idx] = sh_c[qb * NCOL + qj];
    }
  }
}

// ====================================================================== bwd
template <int MODE, bool BF16, int NT, int MT, int KPW, int NW>
__global__ __launch_bounds__(NW * 64) void rnn_bwd_kernel(const BwdParams p) {
  constexpr int G = gates_of(MODE);
  constexpr int R = reserve_slots(MODE);
  constexpr int KC = kchunk<BF16>();
  constexpr int PER = KC / 4;
  constexpr int NCOL = NT * 16;
  constexpr int NROW = MT * 16;
  using X = XT<BF16>;

  __shared__ float red[NW][NROW][NCOL + 1];
  __shared__ float sh_dh[NROW * NCOL];
  __shared__ float sh_dc[NROW * NCOL];
  __shared__ int s_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  const int wg = blockIdx.x;
  const int slice = wg % p.nwg;
  const int grp = wg / p.nwg;
  const int c = grp % p.nchunk;
  const int d = grp / p.nchunk;
  const int U = p.U, H = p.H, D = p.D, B = p.B, T = p.T, Hp = p.Hp;
  const int GH = G * H;
  const int KP = G * Hp;
  const int u0 = slice * U;
  const int Uact = min(U, H - u0);
  const int b0 = c * p.Bc;
  const int Bact = min(p.Bc, B - b0);
  const int nch = KP / KC;

  X* xch = reinterpret_cast<X*>(p.xch);
  const size_t gstride = (size_t)2 * p.Bc * KP;
  X* my_x = xch + (size_t)grp * gstride;

  // ---- W_hh^T slice -> registers: B(k = g*Hp + uu, n = j) = W_hh[g*H + uu][u0 + j]
  uint4 wf[KPW][NT];
#pragma unroll
  for (int kk = 0; kk < KPW; ++kk) {
    const int gc = wave + kk * NW;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint32_t v[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) v[e] = 0u;
      const int j = nt * 16 + fr;
      if (gc < nch && j < Uact) {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int k = gc * KC + fq * PER + e;
          const int g = k / Hp, uu = k - g * Hp;
          if (uu < H) v[e] = w_bits<BF16>(p.w_hh, ((size_t)d * GH + (size_t)g * H + uu) * H + u0 + j);
        }
      }
      wf[kk][nt] = pack_frag<BF16>(v);
    }
  }

  const int q = tid;
  const bool qv = q < Bact * Uact;
  const int qb = qv ? q / Uact : 0, qj = qv ? q - (q / Uact) * Uact : 0;
  const int qu = u0 + qj, qbg = b0 + qb;
  const size_t sidx = ((size_t)d * B + qbg) * H + qu;   // [D][B][H] state index
  if (qv) {
    if (p.s_begin == 0) {
      sh_dh[qb * NCOL + qj] = p.dhy ? p.dhy[sidx] : 0.f;
      sh_dc[qb * NCOL + qj] = (MODE == MODE_LSTM && p.dcy) ? p.dcy[sidx] : 0.f;
    } else {
      sh_dh[qb * NCOL + qj] = p.st_dh[sidx];
      if (MODE == MODE_LSTM) sh_dc[qb * NCOL + qj] = p.st_dc[sidx];
    }
  }
  __syncthreads();
  int wgroups[3] = {grp, 0, 0};

  const size_t ystride_t = (size_t)B * D * H;
  for (int s = p.s_begin; s < p.s_end; ++s) {
    const bool final_phase = (s == T);
    const int t = (d == 0) ? T - 1 - s : s;
    // prefetch epilogue inputs
    float dyv = 0.f, rv[5] = {0.f, 0.f, 0.f, 0.f, 0.f}, prevv = 0.f, hcur = 0.f;
    if (!final_phase && qv) {
      dyv = p.dy[(size_t)t * ystride_t + (size_t)qbg * D * H + (size_t)d * H + qu];
      const float* res = p.reserve + (((size_t)d * T + t) * B + qbg) * R * H + qu;
#pragma unroll
      for (int r = 0; r < R; ++r) rv[r] = res[(size_t)r * H];
      const int tp = (d == 0) ? t - 1 : t + 1;
      const bool has_prev = tp >= 0 && tp < T;
      if (MODE == MODE_LSTM) {
        if (has_prev) prevv = p.reserve[(((size_t)d * T + tp) * B + qbg) * R * H + 4 * (size_t)H + qu];
        else prevv = p.c0 ? p.c0[sidx] : 0.f;
      } else if (MODE == MODE_GRU) {
        if (has_prev) prevv = p.y[(size_t)tp * ystride_t + (size_t)qbg * D * H + (size_t)d * H + qu];
        else prevv = p.h0 ? p.h0[sidx] : 0.f;
      } else {
        hcur = p.y[(size_t)t * ystride_t + (size_t)qbg * D * H + (size_t)d * H + qu];
      }
    }

    float dhrec = 0.f;
    if (s > 0) {
      if (p.persistent) {
        if (!wait_groups(p.flags, p.err, p.spin_limit, wgroups, 1, p.nwg, (unsigned)s, &s_flag)) return;
      }
      f32x4 acc[MT][NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const X* src = my_x + (size_t)(s & 1) * p.Bc * KP;
#pragma unroll
      for (int kk = 0; kk < KPW; ++kk) {
        const int gc = wave + kk * NW;
        if (gc < nch) {
          const int k0 = gc * KC + fq * PER;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int row = mt * 16 + fr;
            uint4 a = make_uint4(0u, 0u, 0u, 0u);
            if (row < Bact) a = *reinterpret_cast<const uint4*>(src + (size_t)row * KP + k0);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma_chunk<BF16>(a, wf[kk][nt], acc[mt][nt]);
          }
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[wave][mt * 16 + fq * 4 + r][nt * 16 + fr] = acc[mt][nt][r];
      __syncthreads();
      if (qv) {
#pragma unroll
        for (int w = 0; w < NW; ++w) dhrec += red[w][qb][qj];
      }
    }

    if (qv) {
      const float carry = sh_dh[qb * NCOL + qj];
      if (final_phase) {
        if (p.dh0) p.dh0[sidx] = dhrec + carry;
        if (MODE == MODE_LSTM && p.dc0) p.dc0[sidx] = sh_dc[qb * NCOL + qj];
      } else {
        const float dh = dhrec + dyv + carry;
        float dgi[4] = {0.f, 0.f, 0.f, 0.f}, dgh[4] = {0.f, 0.f, 0.f, 0.f};
        float ncarry = 0.f;
        if (MODE == MODE_LSTM) {
          const float ig = rv[0], fg = rv[1], gg = rv[2], og = rv[3], cc = rv[4];
          const float tau = tanhf(cc);
          const float d_o = dh * tau;
          const float dc = sh_dc[qb * NCOL + qj] + dh * og * (1.f - tau * tau);
          dgi[0] = dc * gg * ig * (1.f - ig);
          dgi[1] = dc * prevv * fg * (1.f - fg);
          dgi[2] = dc * ig * (1.f - gg * gg);
          dgi[3] = d_o * og * (1.f - og);
#pragma unroll
          for (int g = 0; g < 4; ++g) dgh[g] = dgi[g];
          sh_dc[qb * NCOL + qj] = dc * fg;
        } else if (MODE == MODE_GRU) {
          const float rg = rv[0], zg = rv[1], ng = rv[2], ghn = rv[3];
          const float dn = dh * (1.f - zg);
          const float dz = dh * (prevv - ng);
          const float dan = dn * (1.f - ng * ng);
          dgi[0] = dan * ghn * rg * (1.f - rg);
          dgi[1] = dz * zg * (1.f - zg);
          dgi[2] = dan;
          dgh[0] = dgi[0];
          dgh[1] = dgi[1];
          dgh[2] = dan * rg;
          ncarry = dh * zg;
        } else {
          dgi[0] = dh * (1.f - hcur * hcur);
          dgh[0] = dgi[0];
        }
        sh_dh[qb * NCOL + qj] = ncarry;
        const size_t row = ((size_t)t * B + qbg) * D * GH + (size_t)d * GH + qu;
        X* xo = my_x + (size_t)((s + 1) & 1) * p.Bc * KP + (size_t)qb * KP + qu;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          p.dgi[row + (size_t)g * H] = dgi[g];
          if (MODE == MODE_GRU) p.dgh[row + (size_t)g * H] = dgh[g];
          xo[(size_t)g * Hp] = to_x<BF16>(dgh[g]);
        }
      }
    }
    if (p.persistent && !final_phase) publish(p.flags, (unsigned)(s + 1));
    __syncthreads();
  }
  if (qv && p.s_end <= T) {
    p.st_dh[sidx] = sh_dh[qb * NCOL + qj];
    if (MODE == MODE_LSTM) p.st_dc[sidx] = sh_dc[qb * NCOL + qj];
  }
}

// ===================================================================== misc
struct FillArgs {
  void* p[8];
  size_t n[8];   // bytes (multiple of 4)
  int count;
};

__global__ void fill_zero_kernel(const FillArgs a) {
  for (int i = 0; i < a.count; ++i) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.p[i]);
    const size_t nw = a.n[i] / 4;
    for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < nw; k += (size_t)gridDim.x * blockDim.x)
      dst[k] = 0u;
  }
}

__global__ void copy_kernel(float* dst, const float* src, size_t n) {
  for (size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (size_t)gridDim.x * blockDim.x)
    dst[k] = src ? src[k] : 0.f;
}

// -------------------------------------------------------------- dispatch
template <int MODE, bool BF16, int NT, int MT, int KPW, int NW>
struct FwdK {
  static const void* fn() { return reinterpret_cast<const void*>(&rnn_fwd_kernel<MODE, BF16, NT, MT, KPW, NW>); }
  static hipError_t launch(const FwdParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((rnn_fwd_kernel<MODE, BF16, NT, MT, KPW, NW>), dim3(grid), dim3(NW * 64), 0, s, p);
    return hipGetLastError();
  }
};
template <int MODE, bool BF16, int NT, int MT, int KPW, int NW>
struct BwdK {
  static const void* fn() { return reinterpret_cast<const void*>(&rnn_bwd_kernel<MODE, BF16, NT, MT, KPW, NW>); }
  static hipError_t launch(const BwdParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((rnn_bwd_kernel<MODE, BF16, NT, MT, KPW, NW>), dim3(grid), dim3(NW * 64), 0, s, p);
    return hipGetLastError();
  }
};

// Supported configurations (nt, mt, kpw, nwaves).
#define RNN_FWD_CONFIGS(X, M, BF) \
  X(M, BF, 1, 1, 8, 4)            \
  X(M, BF, 1, 2, 8, 4)            \
  X(M, BF, 1, 1, 16, 4)           \
  X(M, BF, 1, 2, 16, 4)           \
  X(M, BF, 2, 2, 8, 4)            \
  X(M, BF, 2, 2, 16, 4)           \
  X(M, BF, 4, 2, 8, 8)            \
  X(M, BF, 1, 2, 32, 4)

#define RNN_BWD_CONFIGS(X, M, BF) \
  X(M, BF, 1, 1, 8, 4)            \
  X(M, BF, 1, 2, 8, 4)            \
  X(M, BF, 1, 2, 16, 4)           \
  X(M, BF, 1, 2, 32, 4)           \
  X(M, BF, 1, 2, 16, 8)           \
  X(M, BF, 1, 2, 32, 8)           \
  X(M, BF, 1, 1, 32, 8)

template <class KFN>
int max_resident(const void* f, int nthr) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, nthr, 0) != hipSuccess) return 0;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return per_cu * ncu;
}

}  // namespace

#define RNN_MATCH(c, NT_, MT_, KPW_, NW_) ((c).nt == NT_ && (c).mt == MT_ && (c).kpw == KPW_ && (c).nwaves == NW_)

#define FWD_LAUNCH_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return FwdK<M, BF, NT_, MT_, KPW_, NW_>::launch(p, grid, s);
#define FWD_RES_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return max_resident<void>(FwdK<M, BF, NT_, MT_, KPW_, NW_>::fn(), NW_ * 64);
#define FWD_SUP_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return true;
#define BWD_LAUNCH_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return BwdK<M, BF, NT_, MT_, KPW_, NW_>::launch(p, grid, s);
#define BWD_RES_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return max_resident<void>(BwdK<M, BF, NT_, MT_, KPW_, NW_>::fn(), NW_ * 64);
#define BWD_SUP_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return true;

#define RNN_ALL_MODES(CFG, X) \
  CFG(X, MODE_TANH, false) CFG(X, MODE_TANH, true) CFG(X, MODE_LSTM, false) CFG(X, MODE_LSTM, true) \
  CFG(X, MODE_GRU, false) CFG(X, MODE_GRU, true)

hipError_t rnn_launch_fwd(const FwdParams& p, int mode, int bf16, const RecConfig& c, int grid,
                          hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  RNN_ALL_MODES(RNN_FWD_CONFIGS, FWD_LAUNCH_CASE)
  return hipErrorInvalidValue;
}
int rnn_fwd_max_resident(int mode, int bf16, const RecConfig& c) {
  RNN_ALL_MODES(RNN_FWD_CONFIGS, FWD_RES_CASE)
  return 0;
}
bool rnn_fwd_config_supported(int mode, int bf16, const RecConfig& c) {
  RNN_ALL_MODES(RNN_FWD_CONFIGS, FWD_SUP_CASE)
  return false;
}
hipError_t rnn_launch_bwd(const BwdParams& p, int mode, int bf16, const RecConfig& c, int grid,
                          hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  RNN_ALL_MODES(RNN_BWD_CONFIGS, BWD_LAUNCH_CASE)
  return hipErrorInvalidValue;
}
int rnn_bwd_max_resident(int mode, int bf16, const RecConfig& c) {
  RNN_ALL_MODES(RNN_BWD_CONFIGS, BWD_RES_CASE)
  return 0;
}
bool rnn_bwd_config_supported(int mode, int bf16, const RecConfig& c) {
  RNN_ALL_MODES(RNN_BWD_CONFIGS, BWD_SUP_CASE)
  return false;
}

hipError_t rnn_launch_fill(void* const* ptrs, const size_t* bytes, int n, hipStream_t s) {
  FillArgs a{};
  size_t total = 0;
  int k = 0;
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i] || bytes[i] == 0) continue;
    if (k == 8) return hipErrorInvalidValue;
    a.p[k] = ptrs[i];
    a.n[k] = bytes[i];
    total += bytes[i];
    ++k;
  }
  a.count = k;
  if (k == 0) return hipSuccess;
  size_t blocks = (total / 4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t rnn_copy_state(float* dst, const float* src, size_t n, hipStream_t s) {
  if (!dst || n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}
