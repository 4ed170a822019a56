// Persistent recurrent sweeps of the GRU flavours whose candidate reads
// (r*h) W_hn (gfx950): the TensorFlow flavour, n = tanh(W_in x + b_in +
// (r*h_prev) W_hn^T + b_hn), h = (1-z) n + z h_prev, and the original-paper
// flavour, the same n with h = (1-z) h_prev + z n (both listed in oneDNN
// issue #218, "GRU flavours").  r must be known for every unit before the n
// product can start, so each step needs two all-to-all exchanges instead of
// one: h, then r*h.  The backward sweep likewise exchanges da_n (for
// d(r*h) = da_n W_hn) and then [da_r, da_z] (for the dh recurrence).
//
// The structure is that of the PyTorch-flavour kernels in recurrent.hip (one
// workgroup per U hidden units, weights resident in VGPRs as MFMA B
// fragments, per-wave waits on the producers' flags, granule-layout exchange
// rings written once per step with agent-scope stores), with two rings per
// group and two flag publications per step: the flag of a workgroup counts
// half-steps.  Persistent launches only.
#include "device_util.h"
#include "recurrent_util.h"
#include "rnn_common.h"

using namespace rnnk;

namespace {

// ====================================================================== fwd
template <bool BF16, int NT, int MT, int KPW, int NW>
__global__ __launch_bounds__(NW * 64) void gru2_fwd_kernel(const FwdParams p) {
  constexpr int G = 3;
  constexpr int R = 4;   // reserve: r, z, n, r*h_prev
  constexpr int PER = kchunk<BF16>() / 4;
  constexpr int NCOL = NT * 16;
  constexpr int NROW = MT * 16;
  constexpr int ES = BF16 ? 2 : 4;

  // per-wave partial tiles, laid out so that the four row groups of one
  // write instruction fall in distinct 16-bank groups: four 16-column tiles
  // and one row tile -- unpadded rows, the 16-column group XORed with
  // (row ^ row / 4) % 4; one or two column tiles and one row tile -- rows
  // padded by 4 floats; otherwise a padding of 1
  constexpr bool RSWZ = NT == 4 && MT == 1;
  __shared__ float red[NW][NROW][RSWZ ? NCOL : (MT == 1 ? NCOL + 4 : NCOL + 1)];
  auto rcol = [](int row, int col) {
    if constexpr (RSWZ) return col ^ ((((row ^ (row >> 2)) & 3)) << 4);
    else return col;
  };
  __shared__ int s_fail;

  // the wave index is the same in every lane: a scalar register keeps the
  // wave's K range, loop bounds and branches scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fq = lane >> 4;
  const int wg = logical_wg(p.place, p.nwg, p.ngroups);
  if (wg < 0) return;   // an idle slot of the XCD-local placement
  const int slice = wg % p.nwg;
  const int grp = wg / p.nwg;
  const int c = grp % p.nchunk;
  const int d = grp / p.nchunk;
  const int layer = p.first_layer;
  const int U = p.U, H = p.H, D = p.D, B = p.B, T = p.T;
  const int GH = G * H;
  const int u0 = slice * U;
  const int Uact = max(0, min(U, H - u0));
  const int b0 = c * p.Bc;
  const int Bact = min(p.Bc, B - b0);
  const int gran = p.gran;
  const int rmax = (gran >> 4) - 1;

  // K = h (or r*h) in unit order, PER units per granule; this wave holds
  // granules [g0, g1), produced by workgroups [ha0, ha0 + hn)
  const int UJ = U / PER;
  const int ngr = p.nwg * UJ;
  const int g0 = (wave * ngr) / NW, g1 = ((wave + 1) * ngr) / NW;
  const int nmine = g1 - g0;
  const int ha0 = nmine > 0 ? g0 / UJ : 0;
  const int hn = nmine > 0 ? (g1 - 1) / UJ + 1 - ha0 : 0;
  const int hflag0 = grp * p.nwg + ha0;

  char* ring = reinterpret_cast<char*>(p.xch) + (size_t)grp * p.ring_group;     // h
  char* ring2 = reinterpret_cast<char*>(p.xch2) + (size_t)grp * p.ring_group;   // r*h
  const void* whh = p.w_hh[0];

  // ---- W_hh slice: columns gb*U + j of gate gb (r, z, n) for the own units
  uint4 wf[KPW][NT];
#pragma unroll
  for (int kk = 0; kk < KPW; ++kk) {
    const int gl = kk * 4 + fq;
    const int kbase = (g0 + gl) * PER;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint32_t v[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) v[e] = 0u;
      const int n = nt * 16 + fr;
      const int gb = n / U, j = n - gb * U;
      if (gl < nmine && gb < G && j < Uact) {
        const size_t row = (size_t)d * GH + (size_t)gb * H + u0 + j;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int k = kbase + e;
          if (k < H) v[e] = w_bits<BF16>(whh, row * H + k);
        }
      }
      wf[kk][nt] = pack_frag<BF16>(v);
    }
  }

  const int q = tid;
  const bool qw = q < Bact * U;
  const int qb = qw ? q / U : 0, qj = qw ? q - (q / U) * U : 0;
  const bool qv = qw && qj < Uact;
  const int qu = u0 + qj, qbg = b0 + qb;
  const size_t hx_idx = (((size_t)layer * D + d) * B + qbg) * H + qu;
  const size_t my_off = (size_t)(slice * UJ + qj / PER) * gran + qb * 16 + (qj % PER) * ES;
  const int qlen = (p.lengths && qv) ? min(max(p.lengths[qbg], 0), T) : T;
  const float bhn = qv ? p.b_hh[0][(size_t)d * GH + 2 * H + qu] : 0.f;

  // the state h of (qb, qj) lives in its owning thread's registers: no
  // other thread reads it
  float hst = 0.f;
  if (tid == 0) s_fail = 0;
  {
    float hv = 0.f;
    if (qv) {
      hv = p.h0 ? p.h0[hx_idx] : 0.f;
      hst = hv;
    }
    if (qw) ring_store<BF16>(ring, my_off, hv);
    publish(p.flags, wg, 1u);
  }
  __syncthreads();

  // one exchange: wait for the producers of this wave's granules of entry
  // `e`, multiply, sum the waves' partial tiles in `red`; false when a wait
  // expired (every wave then leaves after the same barrier)
  auto exchange = [&](const char* e, unsigned target) -> bool {
    f32x4 acc[MT][NT];
    const bool ok = wave_wait(p.flags, p.err, p.spin_limit, hflag0, hn, 0, 0, target);
    if (ok) {
      // the read offset passes through an asm statement after the wait
      int g0s = g0;
      asm volatile("" : "+v"(g0s));
      mfma_sweep<BF16, NT, MT, KPW, (NW >= 8 ? 4 : 8)>(acc, wf, fr, fq, nmine, rmax, [&](int gl, int row) -> uint4 {
        return *reinterpret_cast<const uint4*>(e + (size_t)(g0s + gl) * gran + row * 16);
      });
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (lane == 0) s_fail = 1;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = mt * 16 + fq * 4 + r;
          red[wave][row][rcol(row, nt * 16 + fr)] = acc[mt][nt][r];
        }
    lds_barrier();
    return s_fail == 0;
  };
  auto reduce = [&](int gb) {
    // every wave's partial issued before the first sum
    float part[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) part[w] = red[w][qb][rcol(qb, gb * U + qj)];
    __builtin_amdgcn_sched_barrier(0);
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += part[w];
    return v;
  };

  const size_t ystride_t = (size_t)B * D * H;
  for (int s = 0; s < T; ++s) {
    const int t = (d == 0) ? s : T - 1 - s;
    float gxl[3] = {0.f, 0.f, 0.f};
    if (qv) {
      const float* g = p.gx + ((size_t)t * B + qbg) * D * GH + (size_t)d * GH + qu;
#pragma unroll
      for (int gi = 0; gi < G; ++gi) gxl[gi] = g[(size_t)gi * H];
    }
    // (1) h -> r, z
    if (!exchange(ring + (size_t)s * p.ring_step, (unsigned)(2 * s + 1))) return;
    const float hprev = hst;
    float rg = 0.f, zg = 0.f, rh = 0.f;
    if (qv) {
      rg = sigmoidf_(reduce(0) + gxl[0]);
      zg = sigmoidf_(reduce(1) + gxl[1]);
      rh = rg * hprev;
    }
    if (qw) ring_store<BF16>(ring2 + (size_t)s * p.ring_step, my_off, rh);
    publish(p.flags, wg, (unsigned)(2 * s + 2));
    // (2) r*h -> n, h
    if (!exchange(ring2 + (size_t)s * p.ring_step, (unsigned)(2 * s + 2))) return;
    float hnew = 0.f, ng = 0.f;
    const bool tv = t < qlen;
    if (qv) {
      ng = tanhf_(gxl[2] + reduce(2) + bhn);
      hnew = p.paper ? (1.f - zg) * hprev + zg * ng : (1.f - zg) * ng + zg * hprev;
      if (!tv) hnew = hprev;
      hst = hnew;
    }
    if (qw) ring_store<BF16>(ring + (size_t)(s + 1) * p.ring_step, my_off, hnew);
    publish(p.flags, wg, (unsigned)(2 * s + 3));
    if (qv) {
      p.y[0][(size_t)t * ystride_t + (size_t)qbg * D * H + (size_t)d * H + qu] = tv ? hnew : 0.f;
      if (p.training) {
        float* res = p.reserve[0] + (((size_t)d * T + t) * B + qbg) * R * H + qu;
        res[0] = rg;
        res[H] = zg;
        res[2 * (size_t)H] = ng;
        res[3 * (size_t)H] = rh;
      }
    }
    lds_barrier();   // red is reused by the next step
  }
  if (qv && p.hy) p.hy[hx_idx] = hst;
}

// ====================================================================== bwd
template <bool BF16, int NT, int MT, int KPW, int NW>
__global__ __launch_bounds__(NW * 64) void gru2_bwd_kernel(const BwdParams p) {
  constexpr int G = 3;
  constexpr int R = 4;
  constexpr int PER = kchunk<BF16>() / 4;
  constexpr int NCOL = NT * 16;
  constexpr int NROW = MT * 16;
  constexpr int ES = BF16 ? 2 : 4;

  // rows padded by 4 floats with one row tile: the four row groups of one
  // write instruction fall in distinct 16-bank groups
  __shared__ float red[NW][NROW][MT == 1 ? NCOL + 4 : NCOL + 1];
  __shared__ int s_fail;

  // the wave index is the same in every lane: a scalar register keeps the
  // wave's K range, loop bounds and branches scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fq = lane >> 4;
  const int wg = logical_wg(p.place, p.nwg, p.ngroups);
  if (wg < 0) return;   // an idle slot of the XCD-local placement
  const int slice = wg % p.nwg;
  const int grp = wg / p.nwg;
  const int c = grp % p.nchunk;
  const int d = grp / p.nchunk;
  const int U = p.U, H = p.H, D = p.D, B = p.B, T = p.T;
  const int GH = G * H;
  const int u0 = slice * U;
  const int Uact = max(0, min(U, H - u0));
  const int b0 = c * p.Bc;
  const int Bact = min(p.Bc, B - b0);
  const int UJ = U / PER;

  // exchange A: da_n, one gate per producer slice (granule pp*UJ + jb);
  // exchange B: [da_r, da_z], two gates (granule pp*2UJ + g*UJ + jb)
  const int granA = p.gran, granB = p.gran2;
  const int rmaxA = (granA >> 4) - 1, rmaxB = (granB >> 4) - 1;
  const int ngrA = p.nwg * UJ, ngrB = p.nwg * 2 * UJ;
  const int gA0 = (wave * ngrA) / NW, gA1 = ((wave + 1) * ngrA) / NW, nA = gA1 - gA0;
  const int gB0 = (wave * ngrB) / NW, gB1 = ((wave + 1) * ngrB) / NW, nB = gB1 - gB0;
  const int pA0 = nA > 0 ? gA0 / UJ : 0, pnA = nA > 0 ? (gA1 - 1) / UJ + 1 - pA0 : 0;
  const int pB0 = nB > 0 ? gB0 / (2 * UJ) : 0, pnB = nB > 0 ? (gB1 - 1) / (2 * UJ) + 1 - pB0 : 0;
  char* ringA = reinterpret_cast<char*>(p.xch) + (size_t)grp * p.ring_group;
  char* ringB = reinterpret_cast<char*>(p.xch2) + (size_t)grp * p.ring_group2;

  // W_hn^T (exchange A) and [W_hr; W_hz]^T (exchange B) slices:
  // B(k = (g, uu), n = j) = W_hh[g*H + uu][u0 + j].  Exchange A has half
  // the granules of exchange B, so half the chunks hold all of its share.
  constexpr int KPWA = KPW / 2;
  uint4 wfA[KPWA][NT], wfB[KPW][NT];
#pragma unroll
  for (int kk = 0; kk < KPW; ++kk) {
    const int gl = kk * 4 + fq;
    const int giA = gA0 + gl;
    const int ppA = giA / UJ, ubA = ppA * U + (giA - ppA * UJ) * PER;
    const int giB = gB0 + gl;
    const int ppB = giB / (2 * UJ), remB = giB - ppB * 2 * UJ;
    const int gB = remB / UJ, ubB = ppB * U + (remB - gB * UJ) * PER;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint32_t va[PER], vb[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) va[e] = vb[e] = 0u;
      const int j = nt * 16 + fr;
      if (j < Uact) {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          if (gl < nA && ubA + e < H)
            va[e] = w_bits<BF16>(p.w_hh, ((size_t)d * GH + 2 * (size_t)H + ubA + e) * H + u0 + j);
          if (gl < nB && ubB + e < H)
            vb[e] = w_bits<BF16>(p.w_hh, ((size_t)d * GH + (size_t)gB * H + ubB + e) * H + u0 + j);
        }
      }
      if (kk < KPWA) wfA[kk][nt] = pack_frag<BF16>(va);
      wfB[kk][nt] = pack_frag<BF16>(vb);
    }
  }

  const int q = tid;
  const bool qw = q < Bact * U;
  const int qb = qw ? q / U : 0, qj = qw ? q - (q / U) * U : 0;
  const bool qv = qw && qj < Uact;
  const int qu = u0 + qj, qbg = b0 + qb;
  const size_t sidx = ((size_t)d * B + qbg) * H + qu;
  const int qlen = (p.lengths && qv) ? min(max(p.lengths[qbg], 0), T) : T;
  const size_t offA = (size_t)(slice * UJ + qj / PER) * granA + qb * 16 + (qj % PER) * ES;
  const size_t offB = (size_t)(slice * 2 * UJ + qj / PER) * granB + qb * 16 + (qj % PER) * ES;
  if (tid == 0) s_fail = 0;
  // the carried dh of (qb, qj) lives in its owning thread's registers
  float dhst = 0.f;
  if (qv) dhst = p.dhy ? p.dhy[sidx] : 0.f;
  __syncthreads();

  // one exchange over ring entry `e` with weights `wf`
  auto exchange = [&](const auto& wf, const char* e, int gbase, int nmine, int gran, int rmax, int fa0,
                      int fn, unsigned target) -> float {
    constexpr int KW = std::extent<std::remove_reference_t<decltype(wf)>>::value;
    f32x4 acc[MT][NT];
    const bool ok = wave_wait(p.flags, p.err, p.spin_limit, grp * p.nwg + fa0, fn, 0, 0, target);
    if (ok) {
      // the read offset passes through an asm statement after the wait
      int gb = gbase;
      asm volatile("" : "+v"(gb));
      mfma_sweep<BF16, NT, MT, KW, (NW >= 8 ? 4 : 8)>(acc, wf, fr, fq, nmine, rmax, [&](int gl, int row) -> uint4 {
        return *reinterpret_cast<const uint4*>(e + (size_t)(gb + gl) * gran + row * 16);
      });
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (lane == 0) s_fail = 1;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][mt * 16 + fq * 4 + r][nt * 16 + fr] = acc[mt][nt][r];
    lds_barrier();
    float v = 0.f;
    if (qv) {
      // every wave's partial issued before the first sum
      float part[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) part[w] = red[w][qb][qj];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int w = 0; w < NW; ++w) v += part[w];
    }
    return v;
  };

  const size_t ystride_t = (size_t)B * D * H;
  for (int s = 0; s <= T; ++s) {
    const bool final_phase = (s == T);
    const int t = (d == 0) ? T - 1 - s : s;
    float dyv = 0.f, rg = 0.f, zg = 0.f, ng = 0.f, hp = 0.f;
    if (!final_phase && qv) {
      dyv = p.dy[(size_t)t * ystride_t + (size_t)qbg * D * H + (size_t)d * H + qu];
      const float* res = p.reserve + (((size_t)d * T + t) * B + qbg) * R * H + qu;
      rg = res[0];
      zg = res[H];
      ng = res[2 * (size_t)H];
      const int tp = (d == 0) ? t - 1 : t + 1;
      if (tp >= 0 && tp < qlen) hp = p.y[(size_t)tp * ystride_t + (size_t)qbg * D * H + (size_t)d * H + qu];
      else hp = p.h0 ? p.h0[sidx] : 0.f;
    }
    // (B) dh recurrence from the previous step's [da_r, da_z]
    float dhrec = 0.f;
    if (s > 0) {
      dhrec = exchange(wfB, ringB + (size_t)s * p.ring_step2, gB0, nB, granB, rmaxB, pB0, pnB,
                       (unsigned)(2 * s));
      if (s_fail) return;
    }
    if (final_phase) {
      if (qv && p.dh0) p.dh0[sidx] = dhrec + dhst;
      break;
    }
    const bool tv = t < qlen;
    const float dh = dhrec + (tv ? dyv : 0.f) + dhst;
    float dn, dz, direct;
    if (p.paper) { dn = dh * zg; dz = dh * (ng - hp); direct = dh * (1.f - zg); }
    else { dn = dh * (1.f - zg); dz = dh * (hp - ng); direct = dh * zg; }
    float dan = tv ? dn * (1.f - ng * ng) : 0.f;
    if (qw) ring_store<BF16>(ringA + (size_t)s * p.ring_step, offA, qv ? dan : 0.f);
    publish(p.flags, wg, (unsigned)(2 * s + 1));
    // (A) d(r*h) = da_n W_hn for the own units
    const float drh = exchange(wfA, ringA + (size_t)s * p.ring_step, gA0, nA, granA, rmaxA, pA0, pnA,
                               (unsigned)(2 * s + 1));
    if (s_fail) return;
    float dar = 0.f, daz = 0.f, carry = dh;
    if (tv) {
      dar = drh * hp * rg * (1.f - rg);
      daz = dz * zg * (1.f - zg);
      carry = direct + drh * rg;
    }
    if (qv) dhst = carry;
    if (qw) {
      char* en = ringB + (size_t)(s + 1) * p.ring_step2;
      ring_store<BF16>(en, offB, qv ? dar : 0.f);
      ring_store<BF16>(en, offB + (size_t)UJ * granB, qv ? daz : 0.f);
    }
    publish(p.flags, wg, (unsigned)(2 * s + 2));
    {
      // gate gradients (dG_i = dG_h) for the dX product (dG, columns gg_col)
      // and the weight-gradient products (dG^T, columns tb_k); units past H
      // (dG) and rows past the batch (dG^T) get zeros
      using X = typename std::conditional<BF16, uint16_t, float>::type;
      const float dgv[3] = {qv ? dar : 0.f, qv ? daz : 0.f, qv ? dan : 0.f};
      if (qw) {
        const size_t rowi = (size_t)t * B + qbg;
#pragma unroll
        for (int g = 0; g < 3; ++g)
          reinterpret_cast<X*>(p.dg)[rowi * p.dg_ld + gg_col(d, slice, g, qj, U, 3, p.nwg)] = to_x<BF16>(dgv[g]);
      }
      const int zq = q - (q / U) * U;
      if ((qv || q < p.Bc * U) && zq < Uact) {
        const int kb = qw ? qb : q / U;
        const size_t kp = (size_t)tb_k(c, t, kb, T, p.Bc);
        const size_t col0 = (size_t)d * GH + u0 + zq;
#pragma unroll
        for (int g = 0; g < 3; ++g)
          reinterpret_cast<X*>(p.dgT)[(col0 + (size_t)g * H) * p.tb_ld + kp] = to_x<BF16>(dgv[g]);
      }
    }
    lds_barrier();   // red is reused by the next step
  }
}

// -------------------------------------------------------------- dispatch
#define GRU2_FWD_CONFIGS(X, BF) \
  X(BF, 1, 1, 8, 4)             \
  X(BF, 1, 2, 8, 4)             \
  X(BF, 1, 1, 16, 4)            \
  X(BF, 1, 2, 16, 4)            \
  X(BF, 2, 1, 8, 4)             \
  X(BF, 2, 2, 8, 4)             \
  X(BF, 2, 1, 16, 4)            \
  X(BF, 2, 2, 16, 4)            \
  X(BF, 4, 1, 4, 8)             \
  X(BF, 4, 2, 4, 8)             \
  X(BF, 4, 1, 8, 8)             \
  X(BF, 4, 2, 8, 8)

#define GRU2_BWD_CONFIGS(X, BF) \
  X(BF, 1, 1, 8, 4)             \
  X(BF, 1, 2, 8, 4)             \
  X(BF, 1, 1, 16, 4)            \
  X(BF, 1, 2, 16, 4)            \
  X(BF, 1, 1, 16, 8)            \
  X(BF, 1, 2, 16, 8)

}  // namespace

#define GRU2_MATCH(c, NT_, MT_, KPW_, NW_) ((c).nt == NT_ && (c).mt == MT_ && (c).kpw == KPW_ && (c).nwaves == NW_)
#define GRU2_FWD_LAUNCH(BF, NT_, MT_, KPW_, NW_)                                                       \
  if ((bf16 != 0) == BF && GRU2_MATCH(c, NT_, MT_, KPW_, NW_)) {                                   \
    hipLaunchKernelGGL((gru2_fwd_kernel<BF, NT_, MT_, KPW_, NW_>), dim3(grid), dim3(NW_ * 64), 0, s, p); \
    return hipGetLastError();                                                                       \
  }
#define GRU2_BWD_LAUNCH(BF, NT_, MT_, KPW_, NW_)                                                       \
  if ((bf16 != 0) == BF && GRU2_MATCH(c, NT_, MT_, KPW_, NW_)) {                                   \
    hipLaunchKernelGGL((gru2_bwd_kernel<BF, NT_, MT_, KPW_, NW_>), dim3(grid), dim3(NW_ * 64), 0, s, p); \
    return hipGetLastError();                                                                       \
  }
#define GRU2_FWD_RES(BF, NT_, MT_, KPW_, NW_)                       \
  if ((bf16 != 0) == BF && GRU2_MATCH(c, NT_, MT_, KPW_, NW_))      \
    return max_resident(reinterpret_cast<const void*>(&gru2_fwd_kernel<BF, NT_, MT_, KPW_, NW_>), NW_ * 64, 0);
#define GRU2_BWD_RES(BF, NT_, MT_, KPW_, NW_)                       \
  if ((bf16 != 0) == BF && GRU2_MATCH(c, NT_, MT_, KPW_, NW_))      \
    return max_resident(reinterpret_cast<const void*>(&gru2_bwd_kernel<BF, NT_, MT_, KPW_, NW_>), NW_ * 64, 0);
#define GRU2_SUP(BF, NT_, MT_, KPW_, NW_) \
  if ((bf16 != 0) == BF && GRU2_MATCH(c, NT_, MT_, KPW_, NW_)) return true;

hipError_t rnn_launch_gru2_fwd(const FwdParams& p, int bf16, const RecConfig& c, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  GRU2_FWD_CONFIGS(GRU2_FWD_LAUNCH, false)
  GRU2_FWD_CONFIGS(GRU2_FWD_LAUNCH, true)
  return hipErrorInvalidValue;
}
hipError_t rnn_launch_gru2_bwd(const BwdParams& p, int bf16, const RecConfig& c, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  GRU2_BWD_CONFIGS(GRU2_BWD_LAUNCH, false)
  GRU2_BWD_CONFIGS(GRU2_BWD_LAUNCH, true)
  return hipErrorInvalidValue;
}
int rnn_gru2_fwd_max_resident(int bf16, const RecConfig& c) {
  GRU2_FWD_CONFIGS(GRU2_FWD_RES, false)
  GRU2_FWD_CONFIGS(GRU2_FWD_RES, true)
  return 0;
}
int rnn_gru2_bwd_max_resident(int bf16, const RecConfig& c) {
  GRU2_BWD_CONFIGS(GRU2_BWD_RES, false)
  GRU2_BWD_CONFIGS(GRU2_BWD_RES, true)
  return 0;
}
bool rnn_gru2_fwd_config_supported(int bf16, const RecConfig& c) {
  GRU2_FWD_CONFIGS(GRU2_SUP, false)
  GRU2_FWD_CONFIGS(GRU2_SUP, true)
  return false;
}
bool rnn_gru2_bwd_config_supported(int bf16, const RecConfig& c) {
  GRU2_BWD_CONFIGS(GRU2_SUP, false)
  GRU2_BWD_CONFIGS(GRU2_SUP, true)
  return false;
}
