// Persistent recurrent sweep kernels of the fused RNN (gfx950): templates
// shared by the per-mode translation units recurrent_<mode>_<fwd|bwd>.hip.
//
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
//   1. each wave waits until the producers of the part of h it multiplies
//      have published the step (per-workgroup flags, agent scope; GX for the
//      step is prefetched first),
//   2. multiplies the 16-row batch tiles of that part of h_prev by its weight
//      slice on MFMA (K split across the waves, partial tiles summed through
//      LDS in a fixed order),
//   3. applies the cell equations to its units in the same kernel (fused
//      point-wise step of the optimisation table) and writes the next h into
//      the exchange ring,
//   4. publishes its flag, then writes y and the training reserve (read only
//      by later kernels, so off the critical path).
// Backward: the same structure walks time in reverse; each workgroup owns U
// units, exchanges the recurrent gate gradients dG_h, computes
// dh = dG_h W_hh for its units on MFMA (each wave first copies its part of
// the exchanged dG_h into LDS with direct global->LDS loads), and applies the
// hand-derived BPTT formulas to the reserved forward intermediates.
//
// Exchange protocol.  The vector one step produces (h, or dG_h) goes into a
// ring with one entry per step, so no address is written twice within a
// sweep.  An entry is a sequence of granules: 16 bytes of consecutive units
// (the A-fragment share of one lane in one MFMA: 8 bf16 or 4 fp32 values) for
// every batch row, [row][16 bytes].  Producer pp owns the consecutive
// granules of its units (per gate in the backward), padded so that its slice
// covers whole 128-byte lines; it writes them with agent-scope stores, waits
// for their completion and then stores its step flag (agent scope).  A wave
// consumes a contiguous range of granules, polls only the flags of their
// producers with agent-scope loads and then reads them with plain loads: no
// cache can hold a stale copy of a line that was never read before its single
// writer completed, so no cache write-back or invalidation is needed per
// step, and the workgroups of one XCD share the entry through L2.
// Every wait is bounded; an expired wait sets the error word and every
// workgroup leaves the sweep.
#pragma once

#include <type_traits>

#include "device_util.h"
#include "philox.h"
#include "recurrent_util.h"
#include "rnn_common.h"

using namespace rnnk;

namespace {

// ====================================================================== fwd
template <int MODE, bool BF16, int NT, int MT, int KPW, int NW>
__global__ __launch_bounds__(NW * 64) void rnn_fwd_kernel(const FwdParams p) {
  constexpr int G = gates_of(MODE);
  constexpr int R = reserve_slots(MODE);
  constexpr int PER = kchunk<BF16>() / 4;   // values per lane per MFMA (16 bytes)
  constexpr int NCOL = NT * 16;
  constexpr int NROW = MT * 16;
  constexpr int ES = BF16 ? 2 : 4;

  // per-wave partial tiles, laid out so that the four row groups one write
  // instruction covers (rows 4*fq + r) fall in distinct 16-bank groups: with
  // four 16-column tiles and one row tile the 16-column group of (row, col)
  // is XORed with (row ^ row / 4) % 4 in unpadded rows (the epilogue's four
  // batch rows then fall apart too; measured 49 % -> 2 % conflict cycles);
  // with one or two column tiles and one row tile rows are padded by 4
  // floats (4 * stride = 16 banks mod 64); with two column tiles and bf16
  // weights the 8-column block of (row, col) in unpadded rows is XORed with
  // (bit 1 of row) | (bit 0 ^ bit 2 of row) << 1, which keeps the two rows
  // of each half-wave write and the four rows of 8 units each half-wave of
  // the epilogue reads per gate in distinct banks (counters: 27 % -> 0 %
  // conflict cycles; the fp32-weight kernel, at the register limit, measured
  // 4 % slower with it and keeps the padding); the two-row-tile kernels,
  // which spill, keep a padding of 1 (slower with the others)
  constexpr bool RSWZ = NT == 4 && MT == 1;
  constexpr bool RSWZ2 = BF16 && NT == 2 && MT == 1;
  constexpr int RSTR = (RSWZ || RSWZ2) ? NCOL : (MT == 1 ? NCOL + 4 : NCOL + 1);
  __shared__ __attribute__((aligned(16))) float red[NW][NROW][RSTR];
  // column order of the products and of red: unit-major (column n is gate
  // n % GB of unit n / GB, so a unit's gates are adjacent and the LSTM
  // epilogue reads them as one 16-byte value per wave) with one row tile;
  // gate-major (gate n / U, unit n % U) with two, whose register-bound
  // kernels spilled more weight fragments into the step loop with the
  // unit-major order (5-layer wavefront sweep 1.81 -> 2.12 ms)
  constexpr bool UMAJ = MT == 1;
  // tanh form (tanhf_): select in general; branch in the two-row-tile
  // kernels and the eight-wave bf16 LSTM one (measured: 5-layer wavefront
  // sweep 1.95 vs 2.03 ms, DS2 LSTM training forward 721 vs 735 us; the
  // others 1-2 % faster with the select)
  constexpr bool TSEL = !(MT == 2 || (MODE == MODE_LSTM && BF16 && NW == 8));
  auto rcol = [](int row, int col) {
    if constexpr (RSWZ) return col ^ ((((row ^ (row >> 2)) & 3)) << 4);
    else if constexpr (RSWZ2) return col ^ ((((row >> 1) & 1) | (((row ^ (row >> 2)) & 1) << 1)) << 3);
    else return col;
  };
  // the per-(row, unit) state h, c of an epilogue thread lives in its own
  // registers (hst, cst below): only the owning thread ever touches it
  __shared__ int s_fail;

  // (a scalar wave index, which helps the backward, measured 2-5 % slower here)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fq = lane >> 4;

  const int wg = logical_wg(p.place, p.nwg, p.ngroups);
  if (wg < 0) return;   // an idle slot of the XCD-local placement
  const int slice = wg % p.nwg;
  const int grp = wg / p.nwg;
  const int c = grp % p.nchunk;
  const int d = (grp / p.nchunk) % p.D;
  const int li = grp / (p.nchunk * p.D);
  const int layer = p.first_layer + li;
  const int U = p.U, H = p.H, D = p.D, B = p.B, T = p.T;
  const int GH = G * H;
  const int u0 = slice * U;
  const int Uact = max(0, min(U, H - u0));
  const int b0 = c * p.Bc;
  const int Bact = min(p.Bc, B - b0);
  const bool inproj = p.wavefront && li > 0;
  const int GB = (MODE == MODE_GRU && inproj) ? 4 : G;   // column blocks
  const int I_l = p.in_l[li];
  const int DC = p.D * p.nchunk;
  const int gran = p.gran;
  const int rmax = (gran >> 4) - 1;   // last (padded) row of a granule

  // K in granules: [the layer below's h (wavefront) | own h], each in unit
  // order, PER units per granule; this wave holds granules [g0, g1)
  const int UJ = U / PER;
  const int ngr_h = p.nwg * UJ;
  const int xoff = inproj ? ngr_h : 0;
  const int ngr = xoff + ngr_h;
  const int g0 = (wave * ngr) / NW, g1 = ((wave + 1) * ngr) / NW;
  const int nmine = g1 - g0;
  // the producers those granules come from
  int xa0 = 0, xn = 0, ha0 = 0, hn = 0;
  if (nmine > 0 && g0 < xoff) {
    xa0 = g0 / UJ;
    xn = (min(g1, xoff) - 1) / UJ + 1 - xa0;
  }
  if (nmine > 0 && g1 > xoff) {
    ha0 = (max(g0, xoff) - xoff) / UJ;
    hn = (g1 - xoff - 1) / UJ + 1 - ha0;
  }
  const int xflag0 = (grp - DC) * p.nwg + xa0, hflag0 = grp * p.nwg + ha0;

  char* ring = reinterpret_cast<char*>(p.xch) + (size_t)grp * p.ring_group;
  // with dropout the layer above reads the dropped copy of this layer's h
  const bool drop_out = p.xch_drop != nullptr && p.wavefront && li + 1 < p.nlayers;
  char* ring_drop = drop_out ? reinterpret_cast<char*>(p.xch_drop) + (size_t)grp * p.ring_group : nullptr;
  const char* ring_below =
      inproj ? reinterpret_cast<const char*>(p.xch_drop ? p.xch_drop : p.xch) + (size_t)(grp - DC) * p.ring_group
             : ring;
  const void* wih = p.w_ih[li];
  const void* whh = p.w_hh[li];

  // ---- weight slice -> registers (B operand fragments)
  uint4 wf[KPW][NT];
  const bool live = !p.probe;   // the exchange probe skips every use of weights and outputs
#pragma unroll
  for (int kk = 0; kk < KPW; ++kk) {
    const int gl = kk * 4 + fq;
    const int gg = g0 + gl;
    const bool xpart = gg < xoff;
    const int kbase = (xpart ? gg : gg - xoff) * PER;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint32_t v[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) v[e] = 0u;
      const int n = nt * 16 + fr;
      int j, gb;
      if constexpr (UMAJ) {
        j = n / GB;
        gb = n - j * GB;
      } else {
        gb = n / U;
        j = n - gb * U;
      }
      if (live && gl < nmine && gb < GB && j < Uact) {
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
          const int k = kbase + e;
          if (xpart) {
            if (use_x && k < I_l) v[e] = w_bits<BF16>(wih, row * I_l + k);
          } else {
            if (use_h && k < H) v[e] = w_bits<BF16>(whh, row * H + k);
          }
        }
      }
      wf[kk][nt] = pack_frag<BF16>(v);
    }
  }

  // ---- epilogue ownership: thread q <-> (row qb, unit qj) over Bact x U
  const int q = tid;
  const bool qw = q < Bact * U;             // writes the ring (zeros for padded units)
  const int qb = qw ? q / U : 0, qj = qw ? q - (q / U) * U : 0;
  const bool qv = qw && qj < Uact;          // a real (row, unit)
  const bool w0 = Bact * U <= 64;           // every ring store is made by wave 0
  const int qu = u0 + qj, qbg = b0 + qb;
  const size_t st_idx = (((size_t)li * D + d) * B + qbg) * H + qu;
  const size_t hx_idx = (((size_t)layer * D + d) * B + qbg) * H + qu;
  const size_t my_off = (size_t)(slice * UJ + qj / PER) * gran + qb * 16 + (qj % PER) * ES;
  // valid steps of this row (t < qlen); past them the state is carried and y is 0
  const int qlen = (p.lengths && qv && live) ? min(max(p.lengths[qbg], 0), T) : T;

  float hst = 0.f, cst = 0.f;   // this thread's h and c
  if (tid == 0) s_fail = 0;
  if (p.s_begin < 0) {
    float hv = 0.f, cv = 0.f;
    if (qv && live) {
      hv = p.h0 ? p.h0[hx_idx] : 0.f;
      cv = (MODE == MODE_LSTM && p.c0) ? p.c0[hx_idx] : 0.f;
      hst = hv;
      cst = cv;
    }
    const int first = p.wavefront ? li : 0;
    if (qw) ring_store<BF16>(ring + (size_t)first * p.ring_step, my_off, hv);
    if (p.persistent) publish(p.flags, wg, 1u);
  } else if (qv && live) {
    hst = p.st_h[st_idx];
    if (MODE == MODE_LSTM) cst = p.st_c[st_idx];
  }
  __syncthreads();

  // biases that stay in the pre-activations over all steps: the input
  // projection's when it is computed here (wavefront layers above the first),
  // and GRU's b_hn otherwise
  float bconst[4] = {0.f, 0.f, 0.f, 0.f};
  float bhn = 0.f;
  if (qv && live) {
    const float* bi = p.b_ih[li] + (size_t)d * GH + qu;
    const float* bh = p.b_hh[li] + (size_t)d * GH + qu;
    if (inproj) {
      if (MODE == MODE_GRU) {
        bconst[0] = bi[0] + bh[0];
        bconst[1] = bi[H] + bh[H];
        bconst[2] = bi[2 * H];   // b_in (x part of n)
        bconst[3] = bh[2 * H];   // b_hn (h part of n)
      } else {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) bconst[gi] = bi[(size_t)gi * H] + bh[(size_t)gi * H];
      }
    } else if (MODE == MODE_GRU) {
      bhn = bh[2 * H];
    }
  }

  const size_t ystride_t = (size_t)B * D * H;
  for (int s = max(p.s_begin, 0); s < p.s_end; ++s) {
    const int t_rel = p.wavefront ? s - li : s;
    const bool active = t_rel >= 0 && t_rel < T;
    const int t = (d == 0) ? t_rel : T - 1 - t_rel;
    if (!active) {   // uniform across the workgroup; still publishes the step
      if (p.persistent) publish(p.flags, wg, (unsigned)(s + 2));
      continue;
    }

    // this step's dropout multiplier for the layer above (data independent,
    // so computed before the wait)
    float dmul = 0.f;
    if (drop_out && qv && live)
      dmul = dropout_mult(((unsigned long long)t * B + qbg) * (unsigned long long)(D * H) + (size_t)d * H + qu,
                          (uint32_t)(layer + 1), p.drop_k0, p.drop_k1, p.drop_thr, p.drop_scale);

    // input part of the pre-activations (independent of other workgroups):
    // issued now, first used in the epilogue, so its latency overlaps the wait
    float gxl[4] = {0.f, 0.f, 0.f, 0.f};
    if (qv && live && !inproj) {
      const float* g = p.gx + ((size_t)t * B + qbg) * D * GH + (size_t)d * GH + qu;
#pragma unroll
      for (int gi = 0; gi < G; ++gi) gxl[gi] = g[(size_t)gi * H];
    }

    // each wave waits only for the producers of its own granules
    f32x4 acc[MT][NT];
    bool ok = true;
    if (p.persistent) {
      if (p.group_poll) {   // wave 0 waits for every producer, the others at the barrier
        if (wave == 0 && !wave_wait(p.flags, p.err, p.spin_limit, (grp - DC) * p.nwg, inproj ? p.nwg : 0,
                                    grp * p.nwg, p.nwg, (unsigned)(s + 1)) && lane == 0)
          s_fail = 1;
        __syncthreads();
        ok = s_fail == 0;
      } else {
        ok = wave_wait(p.flags, p.err, p.spin_limit, xflag0, xn, hflag0, hn, (unsigned)(s + 1));
      }
    }
    if (ok && live) {
      const char* eh = ring + (size_t)s * p.ring_step;
      const char* ex = ring_below + (size_t)s * p.ring_step;
      // the fragment offsets are recomputed every step (a few VALU
      // operations) instead of being held in registers across the sweep;
      // passed through an asm statement after the wait, they also keep every
      // read of the entry behind it
      int g0s = g0;
      asm volatile("" : "+v"(g0s));
      // eight waves share the register file two per SIMD: smaller batches
      constexpr int KBD = NW >= 8 ? 4 : 8;
      mfma_sweep<BF16, NT, MT, KPW, KBD>(acc, wf, fr, fq, nmine, rmax, [&](int gl, int row) -> uint4 {
        const int gg = g0s + gl;
        const bool xpart = gg < xoff;
        return *reinterpret_cast<const uint4*>((xpart ? ex : eh) + (xpart ? gg : gg - xoff) * gran + row * 16);
      });
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (!ok && lane == 0) s_fail = 1;
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
    // The eight-wave LSTM kernels of one row tile read the failure word with
    // the partial sums, not before them, so its LDS round trip overlaps
    // theirs (every wave leaves after the same barrier): DS2 training forward
    // 722 -> 713 us.  The others keep the check first (the reordering moved
    // their register allocation: wavefront sweep 1.84 -> 2.04 ms, GRU
    // forward 684 -> 692 us, four-wave LSTM inference 0.778 -> 0.786 ms).
    constexpr bool EARLY = UMAJ && MODE == MODE_LSTM && RSTR % 4 == 0 && NW == 8;
    float pre_e[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (EARLY) {
      const int failed = s_fail;
      if (qv && live) {
        // the unit's four gates are one 16-byte read per wave, all issued
        // before the first sum
        float4 v4[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) v4[w] = *reinterpret_cast<const float4*>(&red[w][qb][rcol(qb, qj * 4)]);
        __builtin_amdgcn_sched_barrier(0);
        pre_e[0] = v4[0].x;
        pre_e[1] = v4[0].y;
        pre_e[2] = v4[0].z;
        pre_e[3] = v4[0].w;
#pragma unroll
        for (int w = 1; w < NW; ++w) {
          pre_e[0] += v4[w].x;
          pre_e[1] += v4[w].y;
          pre_e[2] += v4[w].z;
          pre_e[3] += v4[w].w;
        }
      }
      if (failed) return;
    } else {
      if (s_fail) return;
    }

    float hnew = 0.f;
    float rv[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
    if (qv && live) {
      float gxv[4];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) gxv[gi] = inproj ? bconst[gi] : gxl[gi];
      float pre[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (EARLY) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) pre[gi] = pre_e[gi];
      } else if constexpr (UMAJ) {
#pragma unroll
        for (int gb = 0; gb < 4; ++gb) {
          if (gb < GB) {
            const int col = rcol(qb, qj * GB + gb);
            pre[gb] = red[0][qb][col];
#pragma unroll
            for (int w = 1; w < NW; ++w) pre[gb] += red[w][qb][col];
          }
        }
      } else {
        // (the two-row-tile kernels sum from zero: seeding from the first
        // wave changed their register allocation, 5-layer wavefront sweep
        // 1.81 -> 1.94 ms)
#pragma unroll
        for (int gb = 0; gb < 4; ++gb) {
          float v = 0.f;
          if (gb < GB) {
#pragma unroll
            for (int w = 0; w < NW; ++w) v += red[w][qb][rcol(qb, gb * U + qj)];
          }
          pre[gb] = v;
        }
      }
      const float hprev = hst;
      const bool tv = t < qlen;
      if (MODE == MODE_LSTM) {
        const float ig = sigmoidf_(pre[0] + gxv[0]);
        const float fg = sigmoidf_(pre[1] + gxv[1]);
        const float gg = tanhf_<TSEL>(pre[2] + gxv[2]);
        const float og = sigmoidf_(pre[3] + gxv[3]);
        const float cprev = cst;
        const float cn = tv ? fg * cprev + ig * gg : cprev;
        hnew = og * tanhf_<TSEL>(cn);
        cst = cn;
        rv[0] = ig; rv[1] = fg; rv[2] = gg; rv[3] = og; rv[4] = cn;
      } else if (MODE == MODE_GRU) {
        const float rg = sigmoidf_(pre[0] + gxv[0]);
        const float zg = sigmoidf_(pre[1] + gxv[1]);
        float ghn, gin;
        if (inproj) { gin = pre[2] + gxv[2]; ghn = pre[3] + gxv[3]; }
        else { gin = gxv[2]; ghn = pre[2] + bhn; }
        const float ng = tanhf_<TSEL>(gin + rg * ghn);
        hnew = (1.f - zg) * ng + zg * hprev;
        rv[0] = rg; rv[1] = zg; rv[2] = ng; rv[3] = ghn;
      } else {
        hnew = tanhf_<TSEL>(pre[0] + gxv[0]);
      }
      if (!tv) hnew = hprev;
      hst = hnew;
    }
    // only the exchange store precedes the flag; y and the reserve are read
    // by later kernels, so they are written after it, off the critical path
    if (qw) ring_store<BF16>(ring + (size_t)(s + 1) * p.ring_step, my_off, hnew);
    if (qw && drop_out) ring_store<BF16>(ring_drop + (size_t)(s + 1) * p.ring_step, my_off, hnew * dmul);
    if (p.persistent) publish(p.flags, wg, (unsigned)(s + 2), w0);
    if (qv && live) {
      p.y[li][(size_t)t * ystride_t + (size_t)qbg * D * H + (size_t)d * H + qu] = t < qlen ? hnew : 0.f;
      if (p.training && R > 0) {
        float* res = p.reserve[li] + (((size_t)d * T + t) * B + qbg) * R * H + qu;
#pragma unroll
        for (int r = 0; r < R; ++r) res[(size_t)r * H] = rv[r];
      }
    }
    lds_barrier();   // red is reused by the next step
  }

  if (qv && live) {
    if (p.s_end >= p.s_total) {
      if (p.hy) p.hy[hx_idx] = hst;
      if (MODE == MODE_LSTM && p.cy) p.cy[hx_idx] = cst;
    } else {
      p.st_h[st_idx] = hst;
      if (MODE == MODE_LSTM) p.st_c[st_idx] = cst;
    }
  }
}

// ====================================================================== bwd
template <int MODE, bool BF16, int NT, int MT, int KPW, int NW>
__global__ __launch_bounds__(NW * 64) void rnn_bwd_kernel(const BwdParams p) {
  constexpr int G = gates_of(MODE);
  constexpr int R = reserve_slots(MODE);
  constexpr int PER = kchunk<BF16>() / 4;
  constexpr int NCOL = NT * 16;
  constexpr int NROW = MT * 16;
  constexpr int ES = BF16 ? 2 : 4;

  // rows padded by 4 floats with one row tile: the four row groups of one
  // write instruction fall in distinct 16-bank groups
  __shared__ float red[NW][NROW][MT == 1 ? NCOL + 4 : NCOL + 1];
  // per-(row, unit) state of the epilogue threads, row-major (with one
  // 16-column tile the rows and units of a wave already fall in distinct banks)
  __shared__ float sh_dh[NROW * NCOL];
  __shared__ float sh_dc[NROW * NCOL];
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
  const int gran = p.gran;
  const int rmax = (gran >> 4) - 1;

  // K in granules: producer slice pp holds (gate g, units pp*U + jb*PER ..)
  // as granule pp*G*UJ + g*UJ + jb; this wave holds granules [g0, g1)
  const int UJ = U / PER;
  const int GU = G * UJ;
  const int ngr = p.nwg * GU;
  const int g0 = (wave * ngr) / NW, g1 = ((wave + 1) * ngr) / NW;
  const int nmine = g1 - g0;
  const int pa0 = g0 / GU;
  const int pn = nmine > 0 ? (g1 - 1) / GU + 1 - pa0 : 0;
  const int flag0 = grp * p.nwg + pa0;

  char* ring = reinterpret_cast<char*>(p.xch) + (size_t)grp * p.ring_group;

  // ---- W_hh^T slice -> registers: B(k = (g, uu), n = j) = W_hh[g*H + uu][u0 + j]
  uint4 wf[KPW][NT];
#pragma unroll
  for (int kk = 0; kk < KPW; ++kk) {
    const int gl = kk * 4 + fq;
    const int gi = g0 + gl;
    const int pp = gi / GU, rem = gi - pp * GU;
    const int g = rem / UJ, jb = rem - g * UJ;
    const int ubase = pp * U + jb * PER;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint32_t v[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) v[e] = 0u;
      const int j = nt * 16 + fr;
      if (gl < nmine && j < Uact) {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int uu = ubase + e;
          if (uu < H) v[e] = w_bits<BF16>(p.w_hh, ((size_t)d * GH + (size_t)g * H + uu) * H + u0 + j);
        }
      }
      wf[kk][nt] = pack_frag<BF16>(v);
    }
  }

  const int q = tid;
  const bool qw = q < Bact * U;
  const int qb = qw ? q / U : 0, qj = qw ? q - (q / U) * U : 0;
  const bool qv = qw && qj < Uact;
  const int shix = qb * NCOL + qj;   // its slot in sh_dh / sh_dc
  const bool w0 = Bact * U <= 64;     // every ring store is made by wave 0
  const int qu = u0 + qj, qbg = b0 + qb;
  const size_t sidx = ((size_t)d * B + qbg) * H + qu;   // [D][B][H] state index
  // valid steps of this row (t < qlen); every step without lengths
  const int qlen = (p.lengths && qv) ? min(max(p.lengths[qbg], 0), T) : T;
  // ring offset of gate 0 of (qb, qj); gate g is g*UJ granules further
  const size_t my_off = (size_t)(slice * GU + qj / PER) * gran + qb * 16 + (qj % PER) * ES;
  if (tid == 0) s_fail = 0;
  if (qv) {
    if (p.s_begin == 0) {
      sh_dh[shix] = p.dhy ? p.dhy[sidx] : 0.f;
      sh_dc[shix] = (MODE == MODE_LSTM && p.dcy) ? p.dcy[sidx] : 0.f;
    } else {
      sh_dh[shix] = p.st_dh[sidx];
      if (MODE == MODE_LSTM) sh_dc[shix] = p.st_dc[sidx];
    }
  }
  __syncthreads();

  const size_t ystride_t = (size_t)B * D * H;
  auto lds = (char __attribute__((address_space(3)))*)(dyn_lds);
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
      // the previous state is h0 / c0 at the row's first step
      const bool has_prev = tp >= 0 && tp < qlen;
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
      f32x4 acc[MT][NT];
      // the entry's address passes through an asm statement after the wait:
      // no read of the entry can be issued before the flags were seen
      long long eoff = (long long)s * p.ring_step;
      // each wave waits only for the producers of its own granules
      bool ok = true;
      if (p.persistent) {
        if (p.group_poll) {
          if (wave == 0 && !wave_wait(p.flags, p.err, p.spin_limit, grp * p.nwg, p.nwg, 0, 0, (unsigned)s) &&
              lane == 0)
            s_fail = 1;
          __syncthreads();
          ok = s_fail == 0;
        } else {
          ok = wave_wait(p.flags, p.err, p.spin_limit, flag0, pn, 0, 0, (unsigned)s);
        }
      }
      asm volatile("" : "+s"(eoff));
      const char* e = ring + eoff;
      if (ok && p.stage) {
        stage_granules(lds, e, g0, nmine, gran, lane);
        // (batches of 32 LDS fragments measured no faster than 8, and 8 keep
        // the register count low enough for two workgroups per CU)
        constexpr int KBL = NW >= 8 ? 4 : 8;
        mfma_sweep<BF16, NT, MT, KPW, KBL>(acc, wf, fr, fq, nmine, rmax,
            [&](int gl, int row) -> uint4 { return lds_load16(lds + (g0 + gl) * gran + row * 16); });
      } else if (ok) {
        constexpr int KBD = NW >= 8 ? 4 : 8;
        mfma_sweep<BF16, NT, MT, KPW, KBD>(acc, wf, fr, fq, nmine, rmax,
            [&](int gl, int row) -> uint4 { return *reinterpret_cast<const uint4*>(e + (g0 + gl) * gran + row * 16); });
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
      // (the failure word is read with the partial sums, so its LDS round
      // trip overlaps theirs; every wave leaves after the same barrier)
      const int failed = s_fail;
      if (qv) {
        // every wave's partial issued before the first sum
        float part[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) part[w] = red[w][qb][qj];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int w = 0; w < NW; ++w) dhrec += part[w];
      }
      if (failed) return;
    }

    float dgi[4] = {0.f, 0.f, 0.f, 0.f}, dgh[4] = {0.f, 0.f, 0.f, 0.f};
    if (final_phase) {
      if (qv) {
        if (p.dh0) p.dh0[sidx] = dhrec + sh_dh[shix];
        if (MODE == MODE_LSTM && p.dc0) p.dc0[sidx] = sh_dc[shix];
      }
    } else {
      if (qv) {
        // a step past the row's length passes dh (and dc) through and
        // ignores dy; its gate gradients stay zero
        const bool tv = t < qlen;
        const float dh = dhrec + (tv ? dyv : 0.f) + sh_dh[shix];
        float ncarry = dh;
        if (!tv) {
        } else if (MODE == MODE_LSTM) {
          ncarry = 0.f;
          const float ig = rv[0], fg = rv[1], gg = rv[2], og = rv[3], cc = rv[4];
          const float tau = tanhf_(cc);
          const float d_o = dh * tau;
          const float dc = sh_dc[shix] + dh * og * (1.f - tau * tau);
          dgi[0] = dc * gg * ig * (1.f - ig);
          dgi[1] = dc * prevv * fg * (1.f - fg);
          dgi[2] = dc * ig * (1.f - gg * gg);
          dgi[3] = d_o * og * (1.f - og);
#pragma unroll
          for (int g = 0; g < 4; ++g) dgh[g] = dgi[g];
          sh_dc[shix] = dc * fg;
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
          ncarry = 0.f;
          dgi[0] = dh * (1.f - hcur * hcur);
          dgh[0] = dgi[0];
        }
        sh_dh[shix] = ncarry;
      }
      // only the exchange stores precede the flag
      if (qw) {
        char* en = ring + (size_t)(s + 1) * p.ring_step;
#pragma unroll
        for (int g = 0; g < G; ++g) ring_store<BF16>(en, my_off + (size_t)g * UJ * gran, dgh[g]);
      }
    }
    if (p.persistent && !final_phase) publish(p.flags, wg, (unsigned)(s + 1), w0);
    if (!final_phase) {
      // gate gradients for the dX product (dG, columns gg_col) and,
      // transposed, for the weight-gradient products (dG^T, columns tb_k):
      // read by later kernels; units past H (dG) and rows past the batch
      // (dG^T) get zeros
      using X = XT<BF16>;
      if (qw) {
        const size_t rowi = (size_t)t * B + qbg;
#pragma unroll
        for (int g = 0; g < G; ++g)
          reinterpret_cast<X*>(p.dg)[rowi * p.dg_ld + gg_col(d, slice, g, qj, U, G, p.nwg)] = to_x<BF16>(dgi[g]);
      }
      const int zq = q - (q / U) * U;
      if ((qv || q < p.Bc * U) && zq < Uact) {
        const int kb = qw ? qb : q / U;   // rows past the batch: zeros
        const size_t kp = (size_t)tb_k(c, t, kb, T, p.Bc);
        const size_t col0 = (size_t)d * GH + u0 + zq;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const size_t col = col0 + (size_t)g * H;
          reinterpret_cast<X*>(p.dgT)[col * p.tb_ld + kp] = to_x<BF16>(qv ? dgi[g] : 0.f);
          if (MODE == MODE_GRU) reinterpret_cast<X*>(p.dghT)[col * p.tb_ld + kp] = to_x<BF16>(qv ? dgh[g] : 0.f);
        }
      }
    }
    lds_barrier();   // red and sh_* are reused by the next step
  }
  if (qv && p.s_end <= T) {
    p.st_dh[sidx] = sh_dh[shix];
    if (MODE == MODE_LSTM) p.st_dc[sidx] = sh_dc[shix];
  }
}

template <int MODE, bool BF16, int NT, int MT, int KPW, int NW>
struct FwdK {
  static const void* fn() { return reinterpret_cast<const void*>(&rnn_fwd_kernel<MODE, BF16, NT, MT, KPW, NW>); }
  static hipError_t launch(const FwdParams& p, int grid, size_t lds, hipStream_t s) {
    if (lds > 0) {
      hipError_t e = hipFuncSetAttribute(fn(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((rnn_fwd_kernel<MODE, BF16, NT, MT, KPW, NW>), dim3(grid), dim3(NW * 64), lds, s, p);
    return hipGetLastError();
  }
};
template <int MODE, bool BF16, int NT, int MT, int KPW, int NW>
struct BwdK {
  static const void* fn() { return reinterpret_cast<const void*>(&rnn_bwd_kernel<MODE, BF16, NT, MT, KPW, NW>); }
  static hipError_t launch(const BwdParams& p, int grid, size_t lds, hipStream_t s) {
    if (lds > 0) {
      hipError_t e = hipFuncSetAttribute(fn(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((rnn_bwd_kernel<MODE, BF16, NT, MT, KPW, NW>), dim3(grid), dim3(NW * 64), lds, s, p);
    return hipGetLastError();
  }
};

// Supported configurations (nt, mt, kpw, nwaves).
#define RNN_FWD_CONFIGS(X, M, BF) \
  X(M, BF, 1, 1, 8, 4)            \
  X(M, BF, 1, 2, 8, 4)            \
  X(M, BF, 1, 1, 16, 4)           \
  X(M, BF, 1, 2, 16, 4)           \
  X(M, BF, 2, 1, 8, 4)            \
  X(M, BF, 2, 2, 8, 4)            \
  X(M, BF, 2, 1, 16, 4)           \
  X(M, BF, 2, 2, 16, 4)           \
  X(M, BF, 4, 1, 4, 8)            \
  X(M, BF, 4, 2, 4, 8)            \
  X(M, BF, 4, 1, 8, 8)            \
  X(M, BF, 4, 2, 8, 8)            \
  X(M, BF, 1, 2, 32, 4)           \
  X(M, BF, 1, 2, 16, 8)           \
  X(M, BF, 2, 2, 16, 8)           \
  X(M, BF, 4, 2, 16, 8)           \
  X(M, BF, 8, 1, 8, 4)

#define RNN_BWD_CONFIGS(X, M, BF) \
  X(M, BF, 1, 1, 8, 4)            \
  X(M, BF, 1, 2, 8, 4)            \
  X(M, BF, 1, 1, 16, 4)           \
  X(M, BF, 1, 2, 16, 4)           \
  X(M, BF, 1, 1, 32, 4)           \
  X(M, BF, 1, 2, 32, 4)           \
  X(M, BF, 1, 1, 16, 8)           \
  X(M, BF, 1, 2, 16, 8)           \
  X(M, BF, 1, 2, 32, 8)           \
  X(M, BF, 1, 1, 32, 8)           \
  X(M, BF, 2, 1, 16, 4)           \
  X(M, BF, 2, 1, 32, 4)           \
  RNN_BWD_WIDE_##BF(X, M)

// 64 K chunks per wave: fp32 only (the bf16 fragments would not fit the
// register file of one wave)
#define RNN_BWD_WIDE_false(X, M) \
  X(M, false, 1, 1, 64, 4)       \
  X(M, false, 1, 2, 64, 4)
#define RNN_BWD_WIDE_true(X, M)


}  // namespace

#define RNN_MATCH(c, NT_, MT_, KPW_, NW_) ((c).nt == NT_ && (c).mt == MT_ && (c).kpw == KPW_ && (c).nwaves == NW_)

#define FWD_LAUNCH_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return FwdK<M, BF, NT_, MT_, KPW_, NW_>::launch(p, grid, lds, s);
#define FWD_RES_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return max_resident(FwdK<M, BF, NT_, MT_, KPW_, NW_>::fn(), NW_ * 64, lds);
#define FWD_SUP_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return true;
#define BWD_LAUNCH_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return BwdK<M, BF, NT_, MT_, KPW_, NW_>::launch(p, grid, lds, s);
#define BWD_RES_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return max_resident(BwdK<M, BF, NT_, MT_, KPW_, NW_>::fn(), NW_ * 64, lds);
#define BWD_SUP_CASE(M, BF, NT_, MT_, KPW_, NW_) \
  if (mode == M && (bf16 != 0) == BF && RNN_MATCH(c, NT_, MT_, KPW_, NW_)) return true;

// Entry points of one cell mode (declared in rnn_common.h), defined in a
// translation unit of their own so that the template instances of the
// modes and directions compile in parallel.
#define RNN_DEFINE_FWD(NAME, M)                                                                       \
  hipError_t rnn_fwd_launch_##NAME(const FwdParams& p, int bf16, const RecConfig& c, int grid, size_t lds, \
                                   hipStream_t s) {                                                    \
    const int mode = M;                                                                               \
    RNN_FWD_CONFIGS(FWD_LAUNCH_CASE, M, false) RNN_FWD_CONFIGS(FWD_LAUNCH_CASE, M, true)               \
    return hipErrorInvalidValue;                                                                      \
  }                                                                                                   \
  int rnn_fwd_resident_##NAME(int bf16, const RecConfig& c, size_t lds) {                             \
    const int mode = M;                                                                               \
    RNN_FWD_CONFIGS(FWD_RES_CASE, M, false) RNN_FWD_CONFIGS(FWD_RES_CASE, M, true)                     \
    return 0;                                                                                         \
  }                                                                                                   \
  bool rnn_fwd_supported_##NAME(int bf16, const RecConfig& c) {                                       \
    const int mode = M;                                                                               \
    RNN_FWD_CONFIGS(FWD_SUP_CASE, M, false) RNN_FWD_CONFIGS(FWD_SUP_CASE, M, true)                     \
    return false;                                                                                     \
  }

#define RNN_DEFINE_BWD(NAME, M)                                                                       \
  hipError_t rnn_bwd_launch_##NAME(const BwdParams& p, int bf16, const RecConfig& c, int grid, size_t lds, \
                                   hipStream_t s) {                                                    \
    const int mode = M;                                                                               \
    RNN_BWD_CONFIGS(BWD_LAUNCH_CASE, M, false) RNN_BWD_CONFIGS(BWD_LAUNCH_CASE, M, true)               \
    return hipErrorInvalidValue;                                                                      \
  }                                                                                                   \
  int rnn_bwd_resident_##NAME(int bf16, const RecConfig& c, size_t lds) {                             \
    const int mode = M;                                                                               \
    RNN_BWD_CONFIGS(BWD_RES_CASE, M, false) RNN_BWD_CONFIGS(BWD_RES_CASE, M, true)                     \
    return 0;                                                                                         \
  }                                                                                                   \
  bool rnn_bwd_supported_##NAME(int bf16, const RecConfig& c) {                                       \
    const int mode = M;                                                                               \
    RNN_BWD_CONFIGS(BWD_SUP_CASE, M, false) RNN_BWD_CONFIGS(BWD_SUP_CASE, M, true)                     \
    return false;                                                                                     \
  }
