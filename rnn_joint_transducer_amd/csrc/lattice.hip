// Lattice recursions and small helper kernels.
//
// Alpha / beta over the transducer lattice (RNN transducer definition on the
// "Daily Papers" page, abstract on sequence transduction with recurrent
// networks; the full sum over alignments, as opposed to the maximum
// approximation discussed in the abstract comparing the two criteria):
//   alpha(0,0) = 0
//   alpha(t,u) = logaddexp(alpha(t-1,u) + LB(t-1,u), alpha(t,u-1) + LE(t,u-1))
//   logP = alpha(T'-1,U') + LB(T'-1,U')
//   beta(T'-1,U') = LB(T'-1,U')
//   beta(t,u) = logaddexp(beta(t+1,u) + LB(t,u), beta(t,u+1) + LE(t,u))
// Maximum approximation (best alignment; same abstract): alpha with max in
// place of logaddexp, the blank predecessor taken on equal scores; the
// predecessor decision of every cell goes to the beta array (1: blank from
// (t-1,u), 2: label from (t,u-1)), and a read-back from (T'-1,U') then marks
// the best alignment's steps there (kPathBlank / kPathLabel).
//
// Cells of one anti-diagonal t+u are independent, so one wave sweeps the
// T'+U' anti-diagonals of an (utterance, direction) with the label positions
// spread over its lanes, while three more waves of its workgroup feed it the
// step weights and store its results.  State is float64, kept in base-2
// units inside the sweep (the posteriors later take exp(alpha + beta - logP)
// of numbers of size ~1e4); the log-add-exp correction log2(1 + 2^-|x-y|)
// lies in [0, 1] and is evaluated in float32.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rnntj {

namespace {

constexpr double kNegInfD = -__builtin_inf();

constexpr double kLog2eD = 1.4426950408889634, kLn2D = 0.6931471805599453;

// Cross-lane shift of a float64 by one lane (DPP wave shifts): shr moves
// lane l-1's value to lane l, shl lane l+1's to lane l; the lane without a
// source (0, resp. 63) receives 0.0.
__device__ __forceinline__ double wave_shr1z(double v) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)x, 0x138, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(x >> 32), 0x138, 0xf, 0xf, true);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ double wave_shl1z(double v) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)x, 0x130, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(x >> 32), 0x130, 0xf, 0xf, true);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// One workgroup of four waves per (utterance, direction); lane l owns the NU
// consecutive label positions u = NU*l .. NU*l + NU-1, so on each
// anti-diagonal the u-1 (alpha) or u+1 (beta) neighbour is in the same lane
// except at the lane edge, which one DPP lane shift supplies.  The
// anti-diagonals go in chunks of CH, and the waves split the work of a chunk
// so that the recursion wave runs nothing but the recursion itself:
//   wave 0   the recursion (two LDS reads, two adds, one log-add-exp and one
//            LDS write per cell),
//   wave 1/2 the step weights of the next chunk: the blank / label
//            log-probabilities loaded, scaled to base 2 and replaced by the
//            finite sentinel kSent wherever the step does not exist,
//   wave 3   the previous chunk's results, scaled back to natural logs and
//            stored (cells outside the lattice are not written).
// With finite sentinels (a weight of -inf is raised to kSent as well) every
// value the recursion meets is finite unless an input is NaN, so the
// log-add-exp needs no guard against -inf - -inf: an impossible step adds
// kSent = -1e300, whose correction
// term rounds to exactly 0, and values near kSent (at most about 7e4 of them
// summed) mark unreachable cells, which are stored as -inf.  The maximum
// approximation (DIR = 2) runs the same scheme with max in place of
// log-add-exp and also hands the predecessor decisions to wave 3.
constexpr double kSent = -1e300;
constexpr double kSentCut = -1e299;  // below: unreachable (-inf)

template <int NU, int CH>
struct LatLds {
  double w[2][2][CH][NU][64];  // [buffer][blank, label][step][slot][lane]
  double r[2][CH][NU][64];     // results (base 2)
  unsigned char dec[2][CH][NU][64];
};

// log2(2^x + 2^y) = max + log2(1 + 2^-|x-y|), the correction in float32.
// A NaN operand makes x - y, and so the result, NaN.
__device__ __forceinline__ double lse2_step(double x, double y) {
  const double m = __builtin_fmax(x, y);
  const float e = (float)(-__builtin_fabs(x - y));
  const float c = __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(e));
  return m + (double)c;
}

template <int DIR, int NU, int CH>
__device__ __forceinline__ void lattice_sweep(LatLds<NU, CH>& sm, const float* __restrict__ LB,
                                              const float* __restrict__ LE,
                                              const int32_t* __restrict__ Teff,
                                              const int32_t* __restrict__ Ueff, const Dims& d,
                                              double* __restrict__ alpha,
                                              double* __restrict__ beta,
                                              double* __restrict__ logP,
                                              float* __restrict__ costs) {
  const int b = blockIdx.x, tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int Tl = Teff[b], Ul = Ueff[b];
  if (Tl == 0) {  // invalid utterance (uniform over the workgroup)
    if (DIR != 1 && tid == 0) {
      costs[b] = __builtin_nanf("");
      logP[b] = __builtin_nan("");
    }
    return;
  }
  constexpr bool kFwd = DIR != 1;
  const int nd = Tl + Ul;  // number of anti-diagonals of this lattice
  const int nch = (nd + CH - 1) / CH;
  const size_t base = (size_t)b * d.DG * d.U1;
  const float* lb = LB + base;
  const float* le = LE + base;
  const int last = d.DG * d.U1 - 1;  // clamp for the loads
  // diagonal of step s
  auto diag = [&](int s) { return kFwd ? s : nd - 1 - s; };

  // waves 1 (K = 0, blank) and 2 (K = 1, label): raw operands of chunk k
  // (clamped, so always in bounds):
  //   alpha: LB(t-1,u), LE(t,u-1) on diagonal dg-1;  beta: LB(t,u), LE(t,u) on dg
  auto load_raw = [&](auto kind, int k, float (&r)[CH][NU]) {
    constexpr int K = decltype(kind)::value;
    const float* src = K ? le : lb;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int dg = diag(k * CH + c);
      const int i0 = (kFwd ? dg - 1 : dg) * d.U1 - ((kFwd && K) ? 1 : 0);
#pragma unroll
      for (int j = 0; j < NU; ++j) {
        const int i = min(max(i0 + NU * l + j, 0), last);
        r[c][j] = src[(unsigned)i];
      }
    }
  };
  // ... and the weights they give, into LDS buffer k & 1
  auto convert = [&](auto kind, int k, const float (&r)[CH][NU]) {
    constexpr int K = decltype(kind)::value;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int dg = diag(k * CH + c);
#pragma unroll
      for (int j = 0; j < NU; ++j) {
        const int u = NU * l + j;
        const int t = dg - u;
        bool ex;
        if (kFwd)
          ex = K ? ((unsigned)t < (unsigned)Tl && u >= 1 && u <= Ul)  // (t,u-1) -> (t,u)
                 : ((unsigned)(t - 1) < (unsigned)(Tl - 1) && u <= Ul);  // (t-1,u) -> (t,u)
        else
          ex = K ? ((unsigned)t < (unsigned)Tl && u < Ul)  // (t,u) -> (t,u+1)
                 : (u <= Ul && ((unsigned)t < (unsigned)(Tl - 1) || (t == Tl - 1 && u == Ul)));
        double v = (double)r[c][j] * kLog2eD;
        v = (ex && !(v < kSent)) ? v : kSent;
        // alpha(0,0) = 0: a zero blank weight from the virtual alpha(-1,0) = 0
        if (kFwd && !K && c == 0)
          if (k == 0) v = u == 0 ? 0.0 : v;
        sm.w[k & 1][K][c][j][l] = v;
      }
    }
  };

  // wave 0: the previous diagonal, in base 2.  It starts as a virtual
  // diagonal with one zero: alpha(-1, 0) (alpha), beta(T', U') behind the
  // final blank (beta).
  double prev[NU];
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    const int u = NU * l + j;
    prev[j] = (DIR == 1 ? u == Ul : u == 0) ? 0.0 : kSent;
  }
  auto recurse = [&](int k) {
    const int q = k & 1;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      // the lane edge gets 0.0: the step from there never exists, so its
      // weight is kSent
      const double edge = kFwd ? wave_shr1z(prev[NU - 1]) : wave_shl1z(prev[0]);
      double res[NU];
#pragma unroll
      for (int j = 0; j < NU; ++j) {
        const double nbv = kFwd ? (j > 0 ? prev[j > 0 ? j - 1 : 0] : edge)
                                : (j + 1 < NU ? prev[j + 1 < NU ? j + 1 : 0] : edge);
        const double ft = prev[j] + sm.w[q][0][c][j][l];
        const double fu = nbv + sm.w[q][1][c][j][l];
        if constexpr (DIR == 2) {
          // best predecessor, blank on equal scores; a NaN operand stays NaN
          const bool pick_t = ft >= fu;
          double v = pick_t ? ft : fu;
          res[j] = (ft != ft || fu != fu) ? ft + fu : v;
          sm.dec[q][c][j][l] = pick_t ? 1 : 2;
        } else {
          res[j] = lse2_step(ft, fu);
        }
      }
#pragma unroll
      for (int j = 0; j < NU; ++j) {
        prev[j] = res[j];
        sm.r[q][c][j][l] = res[j];
      }
    }
  };

  // wave 3: store chunk k (natural logs; unreachable cells -inf; slots
  // outside the lattice go to a per-lane trash slot past the array) and, on
  // the last alpha diagonal, logP = alpha(T'-1,U') + LB(T'-1,U')
  double* arr = DIR == 1 ? beta : alpha;
  double* out = arr + base;
  double* trash = arr + (size_t)d.B * d.DG * d.U1 + NU * l;
  double* dec_out = beta + base;
  double* dec_trash = beta + (size_t)d.B * d.DG * d.U1 + NU * l;
  auto fin = [](double v) { return v < kSentCut ? kNegInfD : v; };
  auto store = [&](int k) {
    const int q = k & 1;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int dg = diag(k * CH + c);
#pragma unroll
      for (int j = 0; j < NU; ++j) {
        const int u = NU * l + j;
        const bool valid = (unsigned)(dg - u) < (unsigned)Tl && u <= Ul;
        const size_t o = (size_t)dg * d.U1 + u;
        *(valid ? out + o : trash + j) = fin(sm.r[q][c][j][l]) * kLn2D;
        if constexpr (DIR == 2) *(valid ? dec_out + o : dec_trash + j) = (double)sm.dec[q][c][j][l];
      }
    }
    if (kFwd && (nd - 1) / CH == k && l == Ul / NU) {
      const double lp =
          (fin(sm.r[q][nd - 1 - k * CH][Ul % NU][l]) +
           (double)lb[(size_t)(nd - 1) * d.U1 + Ul] * kLog2eD) * kLn2D;
      logP[b] = lp;
      costs[b] = (float)(-lp);
    }
  };

  // pipeline: in iteration i wave 0 runs chunk i, waves 1/2 prepare chunk
  // i+1 (loaded in iteration i-1) and load chunk i+2, wave 3 stores chunk
  // i-1; the raw operand registers alternate (no copies)
  using Blank = std::integral_constant<int, 0>;
  using Label = std::integral_constant<int, 1>;
  float ra[CH][NU], rb[CH][NU];
  auto prologue = [&](auto kind) {
    load_raw(kind, 0, ra);
    if (nch > 1) load_raw(kind, 1, rb);
    convert(kind, 0, ra);
  };
  auto produce = [&](auto kind, int i, const float (&cur)[CH][NU], float (&nxt)[CH][NU]) {
    if (i + 2 < nch) load_raw(kind, i + 2, nxt);
    if (i + 1 < nch) convert(kind, i + 1, cur);
  };
  if (w == 1) prologue(Blank{});
  if (w == 2) prologue(Label{});
  __syncthreads();
  auto iter = [&](int i, const float (&cur)[CH][NU], float (&nxt)[CH][NU]) {
    if (w == 0) {
      if (i < nch) recurse(i);
    } else if (w == 1) {
      produce(Blank{}, i, cur, nxt);
    } else if (w == 2) {
      produce(Label{}, i, cur, nxt);
    } else if (i >= 1) {
      store(i - 1);
    }
    __syncthreads();
  };
  for (int i = 0; i <= nch; i += 2) {
    iter(i, rb, ra);
    if (i + 1 <= nch) iter(i + 1, ra, rb);  // uniform
  }
}

// both directions of every utterance in one launch: blockIdx.y = direction
// (full sum); the maximum approximation runs its one forward sweep
template <int NU, int CH, bool MAXA>
__global__ __launch_bounds__(256) void lattice_kernel(const float* __restrict__ LB,
                                                      const float* __restrict__ LE,
                                                      const int32_t* __restrict__ Teff,
                                                      const int32_t* __restrict__ Ueff, Dims d,
                                                      double* __restrict__ alpha,
                                                      double* __restrict__ beta,
                                                      double* __restrict__ logP,
                                                      float* __restrict__ costs) {
  __shared__ LatLds<NU, CH> sm;
  if constexpr (MAXA)
    lattice_sweep<2, NU, CH>(sm, LB, LE, Teff, Ueff, d, alpha, beta, logP, costs);
  else if (blockIdx.y == 0)
    lattice_sweep<0, NU, CH>(sm, LB, LE, Teff, Ueff, d, alpha, beta, logP, costs);
  else
    lattice_sweep<1, NU, CH>(sm, LB, LE, Teff, Ueff, d, alpha, beta, logP, costs);
}

// Maximum approximation: read the best alignment back from (T'-1, U') over
// the predecessor decisions the max-plus pass left in `beta` (1.0: the blank
// step from (t-1,u); anything else: the label step from (t,u-1)), and mark
// each step on the cell it leaves (kPathBlank / kPathLabel).  One workgroup
// per utterance.  Walking back, the path enters row u at some t_hi(u) and
// leaves it at t_lo(u), the highest t <= t_hi(u) whose decision is "label"
// (t = 0 at the latest, where only the label step exists); row 0 runs down to
// t = 0, and t_hi(u-1) = t_lo(u).  So the decisions are packed one bit per
// cell into LDS, row-major in u with t as the bit index (rows S words apart,
// S odd, so that lanes on consecutive u hit distinct banks), and a row's exit
// is a find-last-set over its words (one wave, 64 words a probe).  Utterances
// with more frames than fit are packed in chunks of t from the top, which
// the walk crosses downwards once.  Each anti-diagonal n = t + u holds one
// path cell, in the row u whose [t_lo(u) + u, t_hi(u) + u] contains n, so all
// threads then write the marks at once.
constexpr int kBtThreads = kMaxU1, kBtWords = 8192, kBtBatch = 16;

__global__ __launch_bounds__(kBtThreads) void backtrace_kernel(const int32_t* __restrict__ Teff,
                                                               const int32_t* __restrict__ Ueff,
                                                               Dims d, double* __restrict__ beta) {
  __shared__ uint32_t bits[kBtWords];
  __shared__ int tlo[kMaxU1], thi[kMaxU1];
  __shared__ int s_t, s_u, s_more;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int Tl = Teff[b], Ul = Ueff[b];
  if (Tl == 0) return;  // invalid utterance (uniform over the block)
  const int R = Ul + 1;  // rows u = 0..U'
  // W words (32 W frames) of a row per chunk, rows S = W | 1 words apart;
  // R <= kMaxU1 = 1024 gives W >= 7
  const int W = min((Tl + 31) >> 5, kBtWords / R - 1), S = W | 1;
  const int CT = W * 32;
  if (tid == 0) {
    s_t = Tl - 1;
    s_u = Ul;
    thi[Ul] = Tl - 1;
  }
  const double* ub = beta + (size_t)b * d.DG * d.U1;
  const int q = kBtThreads / R, r = kBtThreads - q * R;
  for (int t1 = Tl;;) {  // chunk: t in [t0, t1)
    const int t0 = max(0, t1 - CT);
    for (int i = tid; i < R * S; i += kBtThreads) bits[i] = 0u;
    __syncthreads();
    // cells of diagonals n in [t0, t1 + U'), u fastest (contiguous in the
    // skewed layout); (no, u) = divmod(i, R) stepped by kBtThreads.  The
    // loads of a batch are unconditional (cells outside the chunk read the
    // utterance's first cell and are dropped), so that they are all in flight
    // together.
    const int nd = t1 - t0 + Ul;
    int no = tid / R, u = tid - (tid / R) * R;
    while (no < nd) {
      double v[kBtBatch];
      int word[kBtBatch];
      uint32_t bit[kBtBatch];
#pragma unroll
      for (int k = 0; k < kBtBatch; ++k) {
        const int t = t0 + no - u;
        const bool ok = no < nd && t >= t0 && t < t1;
        v[k] = ub[ok ? (size_t)(t + u) * d.U1 + u : 0];
        word[k] = u * S + ((t - t0) >> 5);
        bit[k] = ok ? 1u << ((t - t0) & 31) : 0u;
        no += q;
        u += r;
        if (u >= R) {
          u -= R;
          ++no;
        }
      }
#pragma unroll
      for (int k = 0; k < kBtBatch; ++k)
        if (bit[k] != 0u && v[k] != 1.0) atomicOr(&bits[word[k]], bit[k]);
    }
    __syncthreads();
    if (tid < 64) {
      int t = s_t, uu = s_u, more = 0;
      while (uu > 0) {
        const uint32_t* row = bits + uu * S;
        const int w = (t - t0) >> 5, sh = (t - t0) & 31;
        int found = -1;
        for (int wb = w; wb >= 0 && found < 0; wb -= 64) {
          const int wl = wb - lane;
          uint32_t m = 0u;
          if (wl >= 0) {
            m = row[wl];
            if (wl == w && sh < 31) m &= (2u << sh) - 1u;
          }
          const unsigned long long bal = __ballot(m != 0u);
          if (bal) {
            const int L = __builtin_ctzll(bal);  // lowest lane: the highest word
            const uint32_t mw = __shfl(m, L);
            found = t0 + (wb - L) * 32 + (31 - __clz(mw));
          }
        }
        if (found < 0) {
          if (t0 > 0) {  // no label decision in this chunk: continue below it
            t = t0 - 1;
            more = 1;
            break;
          }
          found = 0;
        }
        if (lane == 0) {
          tlo[uu] = found;
          thi[uu - 1] = found;
        }
        t = found;
        --uu;
      }
      if (lane == 0) {
        if (!more) tlo[0] = 0;
        s_t = t;
        s_u = uu;
        s_more = more;
      }
    }
    __syncthreads();
    if (!s_more) break;
    t1 = t0;
  }
  for (int n = tid; n < Tl + Ul; n += kBtThreads) {
    int lo = 0, hi = Ul;  // the largest u with t_lo(u) + u <= n
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tlo[mid] + mid <= n) lo = mid;
      else hi = mid - 1;
    }
    const int t = n - lo;
    beta[skew_idx(d, b, t, lo)] = (lo < Ul && t == thi[lo]) ? kPathLabel : kPathBlank;
  }
}

__global__ void validate_kernel(const int32_t* __restrict__ T_lens,
                                const int32_t* __restrict__ U_lens,
                                const int32_t* __restrict__ labels, Dims d,
                                int32_t* __restrict__ Teff, int32_t* __restrict__ Ueff,
                                int32_t* __restrict__ status, int crit, int32_t tag,
                                int has_logits, int band) {
  __shared__ int sbad;
  const int b = blockIdx.x;
  if (b == 0 && threadIdx.x == 0) {
    status[3] = crit;  // header word 3: the criterion
    status[4] = tag;   // words 4, 5: what a backward from this state must match
    status[5] = has_logits;
    status[kHdrBand] = band;
  }
  if (threadIdx.x == 0) sbad = 0;
  __syncthreads();
  const int Tl = T_lens[b], Ul = U_lens[b];
  int bad = 0;
  if (Tl < 1 || Tl > d.T || Ul < 0 || Ul > d.U) {
    bad = 1;
  } else {
    for (int u = threadIdx.x; u < Ul; u += blockDim.x) {
      const int y = labels[(size_t)b * d.U + u];
      if (y < 0 || y >= d.V || y == d.blank) bad |= 2;
    }
  }
  if (bad) atomicOr(&sbad, bad);
  __syncthreads();
  if (threadIdx.x == 0) {
    Teff[b] = sbad ? 0 : Tl;
    Ueff[b] = sbad ? 0 : Ul;
    if (sbad) atomicOr(status, sbad);
  }
}

// Forward preparation in one launch, three independent jobs by block range:
//   [0, n_tr)            W_out^T, 32 x 32 tiles through LDS;
//   [n_tr, n_tr + n_cb)  the logit bound: for 64 columns v, |b[v]| + sum_k |W[k,v]|,
//                        whose maximum goes to hdr[2] as float bits (non-negative
//                        floats order like their bit patterns; a NaN sum, its sign
//                        bit cleared by fabsf, wins the integer max and disables
//                        the bound); hdr[2] starts at 0;
//   [n_tr + n_cb, ...)   e^{2x} of every enc and pred element (accurate expf) and
//                        the flag that some finite |x| exceeds 40, where e^{2x}
//                        alone could overflow although enc + pred is moderate.
template <typename E>
__global__ __launch_bounds__(256) void prep_kernel(const E* __restrict__ enc,
                                                   const E* __restrict__ pred,
                                                   const E* __restrict__ W,
                                                   const E* __restrict__ bias, Dims d,
                                                   E* __restrict__ Wt, E* __restrict__ Wb,
                                                   float* __restrict__ Eexp,
                                                   float* __restrict__ Pexp,
                                                   int32_t* __restrict__ hdr, int n_tr, int n_cb) {
  __shared__ float sh[32 * 33];
  const int tid = threadIdx.x;
  const int H = d.H, V = d.V;
  int blk = blockIdx.x;
  if (blk < n_tr) {
    E* tile = reinterpret_cast<E*>(sh);  // [32][33]
    const int gx = (V + 31) / 32;
    const int v0 = (blk % gx) * 32, h0 = (blk / gx) * 32;
    const int tx = tid & 31, ty = tid >> 5;  // 32 x 8
    for (int i = ty; i < 32; i += 8) {
      const int h = h0 + i, v = v0 + tx;
      if (h < H) {
        const E x = v < V ? W[(size_t)h * V + v] : E(0);
        if (v < V) tile[i * 33 + tx] = x;
        Wb[((size_t)(v0 >> 5) * H + h) * 32 + tx] = x;  // block v0 / 32, row h, column tx
      }
    }
    __syncthreads();
    for (int i = ty; i < 32; i += 8) {
      const int v = v0 + i, h = h0 + tx;
      if (v < V && h < H) Wt[(size_t)v * H + h] = tile[tx * 33 + i];
    }
    return;
  }
  blk -= n_tr;
  if (blk < n_cb) {
    const int c = tid & 63, g = tid >> 6;
    const int v = blk * 64 + c;
    float s = 0.f;
    if (v < V) {
      // rows g, g+4, ...: eight independent loads in flight per step
      float p[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      int k = g;
      for (; k + 28 < H; k += 32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] += fabsf(ElemTraits<E>::to_f32(W[(size_t)(k + 4 * i) * V + v]));
      }
      for (; k < H; k += 4) p[0] += fabsf(ElemTraits<E>::to_f32(W[(size_t)k * V + v]));
      s = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    }
    sh[g * 64 + c] = s;
    __syncthreads();
    if (g == 0) {
      int m = 0;
      if (v < V)
        m = __float_as_int(sh[c] + sh[64 + c] + sh[128 + c] + sh[192 + c] +
                           fabsf(ElemTraits<E>::to_f32(bias[v])));
      for (int off = 32; off > 0; off >>= 1) m = max(m, __shfl_xor(m, off));
      if (c == 0) atomicMax(&hdr[2], m);
    }
    return;
  }
  blk -= n_cb;
  const size_t ne = (size_t)d.B * d.T * H, np = (size_t)d.B * d.U1 * H;
  const size_t stride = (size_t)(gridDim.x - n_tr - n_cb) * blockDim.x;
  bool bad = false;
  for (size_t i = (size_t)blk * blockDim.x + tid; i < ne + np; i += stride) {
    const float x = i < ne ? ElemTraits<E>::to_f32(enc[i]) : ElemTraits<E>::to_f32(pred[i - ne]);
    const float ax = fabsf(x);
    if (ax > 40.0f && ax != __builtin_inff()) bad = true;
    const float e = expf(2.0f * x);
    if (i < ne)
      Eexp[i] = e;
    else
      Pexp[i - ne] = e;
  }
  if (bad) atomicOr(&hdr[1], kFlagEpBad);
}

// One workgroup per lattice chunk: per-utterance active-tile counts, their
// running offsets, then the packed tile coordinates.
__global__ __launch_bounds__(256) void tile_list_kernel(const int32_t* __restrict__ Teff,
                                                        const int32_t* __restrict__ Ueff, Dims d,
                                                        int CT, int CU, int n_chunks_u, int cap,
                                                        int32_t* __restrict__ list,
                                                        int32_t* __restrict__ count,
                                                        const int32_t* __restrict__ hdr,
                                                        const int32_t* __restrict__ bounds) {
  __shared__ int s_base;
  __shared__ int s_wave[4];
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ct0 = (c / n_chunks_u) * CT, cu0 = (c % n_chunks_u) * CU;
  const int S = hdr ? hdr[kHdrBand] : 0;  // pruning window (0: every tile)
  int32_t* out = list + (size_t)c * cap;
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int b = 0; b < d.B; ++b) {
    const int Tl = Teff[b], Ul = Ueff[b];
    const int tv = min(CT, Tl - ct0), uv = min(CU, Ul + 1 - cu0);
    const int nt = tv > 0 && Tl > 0 ? (tv + kTileT - 1) / kTileT : 0;
    const int nu = uv > 0 ? (uv + kTileU - 1) / kTileU : 0;
    // tiles in order; with a band, a tile is kept when the band's label
    // positions over its frames, [s_first, s_last + S - 1] (s is
    // non-decreasing), meet its own
    for (int i0 = 0; i0 < nt * nu; i0 += 256) {
      const int i = i0 + tid;
      bool keep = i < nt * nu;
      if (keep && S > 0) {
        const int t0 = ct0 + (i / nu) * kTileT, u0 = cu0 + (i % nu) * kTileU;
        const int t1 = min(t0 + kTileT, Tl) - 1, u1 = min(u0 + kTileU - 1, Ul);
        const int32_t* s = bounds + (size_t)b * d.T;
        keep = s[t0] <= u1 && s[t1] + S - 1 >= u0;
      }
      const unsigned long long m = __ballot(keep);
      if (lane == 0) s_wave[w] = __popcll(m);
      __syncthreads();
      int off = s_base;
      for (int k = 0; k < w; ++k) off += s_wave[k];
      const int tot = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
      if (keep) out[off + __popcll(m & ((1ull << lane) - 1ull))] = tile_pack(b, i / nu, i % nu);
      __syncthreads();
      if (tid == 0) s_base += tot;
      __syncthreads();
    }
  }
  if (tid == 0) count[c] = s_base;
}

// Zeroes up to four buffers (32-bit words) in one launch.
struct ZeroList {
  uint32_t* p[4];
  size_t n[4];
};
__global__ void zero_kernel(ZeroList z) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < z.n[k]; i += stride)
      z.p[k][i] = 0u;
}

}  // namespace

hipError_t launch_lattice(const float* LB, const float* LE, const int32_t* Teff,
                          const int32_t* Ueff, const Dims& d, double* alpha, double* beta,
                          double* logP, float* costs, int crit, hipStream_t st) {
  const int nu = (d.U1 + 63) / 64;
  const bool maxa = crit == kCritMax;
  dim3 grid(d.B, maxa ? 1 : 2), block(256);
  // chunk length: about 16 cells per lane and chunk (48 KiB of LDS)
#define RNNTJ_LAT(N, CH)                                                                   \
  case N:                                                                                  \
    if (maxa)                                                                              \
      hipLaunchKernelGGL((lattice_kernel<N, CH, true>), grid, block, 0, st, LB, LE, Teff,  \
                         Ueff, d, alpha, beta, logP, costs);                               \
    else                                                                                   \
      hipLaunchKernelGGL((lattice_kernel<N, CH, false>), grid, block, 0, st, LB, LE, Teff, \
                         Ueff, d, alpha, beta, logP, costs);                               \
    break;
  switch (nu) {
    RNNTJ_LAT(1, 16)
    RNNTJ_LAT(2, 8)
    RNNTJ_LAT(3, 5)
    RNNTJ_LAT(4, 4)
    RNNTJ_LAT(5, 3)
    RNNTJ_LAT(6, 3)
    RNNTJ_LAT(7, 2)
    RNNTJ_LAT(8, 2)
    RNNTJ_LAT(9, 1)
    RNNTJ_LAT(10, 1)
    RNNTJ_LAT(11, 1)
    RNNTJ_LAT(12, 1)
    RNNTJ_LAT(13, 1)
    RNNTJ_LAT(14, 1)
    RNNTJ_LAT(15, 1)
    RNNTJ_LAT(16, 1)
    default:
      return hipErrorInvalidValue;
  }
#undef RNNTJ_LAT
  return hipGetLastError();
}

hipError_t launch_backtrace(const int32_t* Teff, const int32_t* Ueff, const Dims& d, double* beta,
                            hipStream_t st) {
  hipLaunchKernelGGL(backtrace_kernel, dim3(d.B), dim3(kBtThreads), 0, st, Teff, Ueff, d, beta);
  return hipGetLastError();
}

hipError_t launch_tile_list(const int32_t* Teff, const int32_t* Ueff, const Dims& d, int CT, int CU,
                            int n_chunks_u, int n_chunks, int cap, int32_t* list, int32_t* count,
                            const int32_t* hdr, const int32_t* bounds, hipStream_t st) {
  hipLaunchKernelGGL(tile_list_kernel, dim3(n_chunks), dim3(256), 0, st, Teff, Ueff, d, CT, CU,
                     n_chunks_u, cap, list, count, hdr, bounds);
  return hipGetLastError();
}

hipError_t launch_validate(const int32_t* T_lens, const int32_t* U_lens,
                           const int32_t* labels, const Dims& d, int32_t* Teff,
                           int32_t* Ueff, int32_t* status, int crit, int32_t tag,
                           int has_logits, int band, hipStream_t st) {
  hipLaunchKernelGGL(validate_kernel, dim3(d.B), dim3(256), 0, st, T_lens, U_lens, labels, d,
                     Teff, Ueff, status, crit, tag, has_logits, band);
  return hipGetLastError();
}

// A backward checks the state it is given against its own arguments before
// any kernel reads more than the header: on a mismatch it sets kErrPlan and
// the refusal word, which every later kernel of that backward reads first.
__global__ void guard_kernel(int32_t* hdr, int32_t tag, int need_logits) {
  if (threadIdx.x != 0) return;
  const bool ok = hdr[4] == tag && (!need_logits || hdr[5] == 1);
  hdr[kHdrRefuse] = ok ? 0 : 1;
  if (!ok) atomicOr(&hdr[0], kErrPlan);
}

hipError_t launch_guard(int32_t* hdr, int32_t tag, int need_logits, hipStream_t st) {
  hipLaunchKernelGGL(guard_kernel, dim3(1), dim3(64), 0, st, hdr, tag, need_logits);
  return hipGetLastError();
}

hipError_t launch_prep(const void* enc, const void* pred, const void* W, const void* bias,
                       bool bf16, const Dims& d, void* Wt, void* Wb, float* Eexp, float* Pexp,
                       int32_t* hdr, hipStream_t st) {
  const size_t n = (size_t)d.B * (d.T + d.U1) * d.H;
  size_t n_ep = (n + 255) / 256;
  if (n_ep > 8192) n_ep = 8192;
  const int n_tr = ((d.V + 31) / 32) * ((d.H + 31) / 32), n_cb = (d.V + 63) / 64;
  const dim3 grid((unsigned)(n_tr + n_cb + n_ep)), block(256);
  if (bf16)
    hipLaunchKernelGGL(prep_kernel<uint16_t>, grid, block, 0, st, static_cast<const uint16_t*>(enc),
                       static_cast<const uint16_t*>(pred), static_cast<const uint16_t*>(W),
                       static_cast<const uint16_t*>(bias), d, static_cast<uint16_t*>(Wt),
                       static_cast<uint16_t*>(Wb), Eexp, Pexp, hdr, n_tr, n_cb);
  else
    hipLaunchKernelGGL(prep_kernel<float>, grid, block, 0, st, static_cast<const float*>(enc),
                       static_cast<const float*>(pred), static_cast<const float*>(W),
                       static_cast<const float*>(bias), d, static_cast<float*>(Wt),
                       static_cast<float*>(Wb), Eexp, Pexp, hdr, n_tr, n_cb);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t n_words, hipStream_t st) {
  return launch_zero4(p, n_words, nullptr, 0, nullptr, 0, nullptr, 0, st);
}

hipError_t launch_zero4(void* p0, size_t n0, void* p1, size_t n1, void* p2, size_t n2, void* p3,
                        size_t n3, hipStream_t st) {
  ZeroList z = {{static_cast<uint32_t*>(p0), static_cast<uint32_t*>(p1), static_cast<uint32_t*>(p2),
                 static_cast<uint32_t*>(p3)},
                {p0 ? n0 : 0, p1 ? n1 : 0, p2 ? n2 : 0, p3 ? n3 : 0}};
  size_t most = 0;
  for (int k = 0; k < 4; ++k) most = z.n[k] > most ? z.n[k] : most;
  if (most == 0) return hipSuccess;
  size_t blocks = (most + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, z);
  return hipGetLastError();
}

}  // namespace rnntj
