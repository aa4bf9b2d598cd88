// Body of the NNLS solver, included by k_nnls.hip (256 threads per block:
// the LDS-resident refits and the stand-alone solver) and by k_nnls_g.hip
// (512 threads: the workspace-resident refits of large budgets, which are
// bound by the latency of their global-memory passes).  The including file
// defines AMC_NNLS_NT and opens a namespace of its own.
constexpr int NT = AMC_NNLS_NT;  // threads per block (set by the including file)
constexpr bool kGrowBlocks = NT > 256;  // entering blocks grow back (the workspace-resident build)
// Factor rows in fixed slots of mp entries (the workspace-resident build):
// a removal rotates the rows below it in place instead of moving every later
// row up by one.  The LDS build keeps packed rows.
constexpr bool kSlotRows = NT > 256;
constexpr int NW = NT / 64;
constexpr int TB = 16;             // triangular block
constexpr int NB = 8;              // candidates that may enter together
constexpr int NRHS = NB + 1;       // right-hand sides of a block entry (rows 0..8)
constexpr int NROW = NRHS + 2;     // scratch rows: 0 solve vector, 1 change list, 2 scaled change,
                                   // 3 packed scaled change, 4 zero-variable list, 5..6 free,
                                   // 7 removed column, 8 y = L^-1 g_P,
                                   // 9 u at the last snapshot, 10 g at the last snapshot
constexpr unsigned char F_PASSIVE = 1, F_BLOCKED = 2, F_NEW = 4, F_DROP = 8, F_CAND = 16;
constexpr double PIV_TOL = 1e-14;  // smallest acceptable squared pivot in unit-diagonal form
static_assert(NRHS <= 3 * NW, "diagonal solves take three right-hand sides per wave");
static_assert(NRHS == 9, "row roles assume nine right-hand sides");

__device__ __forceinline__ int tri(int r) { return r * (r + 1) / 2; }

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).  Register
// arrays indexed only through it keep constant indices, so they stay in
// registers.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// double broadcast from a (wave-uniform) lane
__device__ __forceinline__ double rl(double x, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
  return __hiloint2double(hi, lo);
}

// Values moved across lanes by a DPP pattern; rows that ROWMASK leaves out
// keep `old`.  The wave reductions below combine lanes within rows of 16
// (quad permutations, the half-row and row mirrors), then row 0 into row 1 and
// row 2 into row 3 (row_bcast:15), then row 1 into rows 2 and 3
// (row_bcast:31): lane 63 holds the result, which v_readlane broadcasts.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ int dpp_i32(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWMASK, 0xf, false);
}
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ double dpp_f64(double old, double v) {
  const int lo = dpp_i32<CTRL, ROWMASK>(__double2loint(old), __double2loint(v));
  const int hi = dpp_i32<CTRL, ROWMASK>(__double2hiint(old), __double2hiint(v));
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<0xB1>(0.0, v);        // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(0.0, v);        // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(0.0, v);       // row_half_mirror
  v += dpp_f64<0x140>(0.0, v);       // row_mirror
  v += dpp_f64<0x142, 0xa>(0.0, v);  // row_bcast:15
  v += dpp_f64<0x143, 0xc>(0.0, v);  // row_bcast:31
  return rl(v, 63);
}

__device__ __forceinline__ int wave_count(int c) {
  c += dpp_i32<0xB1>(0, c);
  c += dpp_i32<0x4E>(0, c);
  c += dpp_i32<0x141>(0, c);
  c += dpp_i32<0x140>(0, c);
  c += dpp_i32<0x142, 0xa>(0, c);
  c += dpp_i32<0x143, 0xc>(0, c);
  return __builtin_amdgcn_readlane(c, 63);
}

// wave-wide best of (v, idx): larger value, ties to the lower index; idx < 0
// is empty
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ void best_step(double &v, int &idx) {
  const double ov = dpp_f64<CTRL, ROWMASK>(v, v);
  const int oi = dpp_i32<CTRL, ROWMASK>(idx, idx);
  if (oi >= 0 && (idx < 0 || ov > v || (ov == v && oi < idx))) {
    v = ov;
    idx = oi;
  }
}
__device__ __forceinline__ void wave_best(double &v, int &idx) {
  best_step<0xB1>(v, idx);
  best_step<0x4E>(v, idx);
  best_step<0x141>(v, idx);
  best_step<0x140>(v, idx);
  best_step<0x142, 0xa>(v, idx);
  best_step<0x143, 0xc>(v, idx);
  v = rl(v, 63);
  idx = __builtin_amdgcn_readlane(idx, 63);
}

struct Red {
  double v[NW];
  int i[NW];
};

// Block max of v (ties to the lower index); returns the winning index, -1 if
// no thread passed a valid one.  Every thread gets the result.
__device__ __forceinline__ int block_argmax(double v, int idx, Red *red, double *out_v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_best(v, idx);
  __syncthreads();
  if (lane == 0) {
    red->v[wave] = v;
    red->i[wave] = idx;
  }
  __syncthreads();
  v = red->v[0];
  idx = red->i[0];
  for (int w = 1; w < NW; ++w) {
    const double ov = red->v[w];
    const int oi = red->i[w];
    if (oi >= 0 && (idx < 0 || ov > v || (ov == v && oi < idx))) {
      v = ov;
      idx = oi;
    }
  }
  *out_v = v;
  return idx;
}

__device__ __forceinline__ int block_count(int c, Red *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  c = wave_count(c);
  __syncthreads();
  if (lane == 0) red->i[wave] = c;
  __syncthreads();
  int s = 0;
  for (int w = 0; w < NW; ++w) s += red->i[w];
  return s;
}

__device__ __forceinline__ double block_sum_d(double v, Red *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red->v[wave] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < NW; ++w) s += red->v[w];
  return s;
}

// Small per-block scratch (always LDS).
struct Blk {
  double dots[NRHS * NRHS];  // Gram of the forward-solved candidate rows (lower triangle)
  double Gc[NB * NB];        // scaled G among the candidates
  double E[NB * NB];         // factor entries among accepted candidates
  double Dg[NB];             // their diagonal
  double yb[NB];             // their entries of L^-1 g
  double cs[2 * TB];         // rotations of one block of the rank-one update
  double xblk[NRHS * TB];    // solved block of the right-hand sides (forward solve)
  int cand[NB];              // entering candidates
  int accb[NB];              // accepted candidates, in order
  int ctl[8];                // [1], [4] scan state, [2] accepted count, [3] largest entering block,
                             // [5] size of the last entering block, [6] an entering variable left
  int wc[NW];                // per-wave counts of a compaction
  int np;                    // free-set size
};

// State of one solve.  Vectors are indexed by variable (u, g, dg, flag, rows
// 9 and 10) or by factor position (plist, the other rows).
struct St {
  double *L;      // packed lower factor of Gs_PP, rows in free-set order
  double *u;      // scaled iterate
  double *g;      // scaled gradient bs - Gs u
  double *dg;     // sqrt(G_aa)
  double *rows;   // NROW scratch rows of mp (roles at NROW)
  double *x0;     // row 0: solve vector (may live apart from rows)
  double *yv;     // row 8: y = L^-1 g_P (may live apart from rows)
  int *plist;     // free set in factor order
  int *slot;      // slot of each factor row (kSlotRows; positions past np hold the free slots)
  unsigned char *flag;
  Blk *bk;
  int mp;         // row stride (largest p of the system)
  bool lds;       // L lives in LDS (the one-wave solves apply up to kWaveRows rows)
  __device__ __forceinline__ double *row(int b) const { return b == 0 ? x0 : (b == 8 ? yv : rows + b * mp); }
  // first element of factor row i (column c of row i is L[rowoff(i) + c])
  __device__ __forceinline__ int rowoff(int i) const {
    if constexpr (kSlotRows)
      return slot[i] * mp;
    else
      return tri(i);
  }
};

// LDS bytes of the state for systems up to maxp variables (LDS variant)
__host__ __device__ constexpr size_t nnls_smem_bytes(int maxp) {
  return size_t(8) * (size_t(maxp) * (maxp + 1) / 2 + size_t(3 + NROW) * maxp) + 4 * size_t(maxp) +
         ((size_t(maxp) + 15) & ~size_t(15));
}

// LDS bytes of the global variant: the two solve vectors, when they fit,
// then the row slots (one int per budget slot).
constexpr int kGlobalLdsRowsMax = 7680;
__host__ __device__ constexpr size_t nnls_global_vec_bytes(int64_t max_t) {
  return max_t <= kGlobalLdsRowsMax ? size_t(16) * size_t(max_t) : 0;
}
__host__ __device__ constexpr size_t nnls_global_smem_bytes(int64_t max_t) {
  return nnls_global_vec_bytes(max_t) + size_t(4) * ((size_t(max_t) + 3) & ~size_t(3));
}

__device__ __forceinline__ St carve_lds(char *base, int maxp, Blk *bk) {
  St s;
  s.mp = maxp;
  s.bk = bk;
  s.lds = true;
  double *d = reinterpret_cast<double *>(base);
  s.L = d;
  d += tri(maxp);
  s.u = d;
  d += maxp;
  s.g = d;
  d += maxp;
  s.dg = d;
  d += maxp;
  s.rows = d;
  s.x0 = d;
  s.yv = d + 8 * maxp;
  d += NROW * maxp;
  s.slot = nullptr;
  s.plist = reinterpret_cast<int *>(d);
  s.flag = reinterpret_cast<unsigned char *>(s.plist + maxp);
  return s;
}

// Global-memory state of one head: u, g, dg, the scratch rows, then the flag
// bytes (and after them, from the next 16-byte boundary, the row slots kept
// between refits); the solve vectors go to LDS (lds, 2 mp doubles) when
// given, the working copy of the row slots to slot_lds.
__host__ __device__ inline int32_t *persisted_slots(double *vec, int mp) {
  return reinterpret_cast<int32_t *>(reinterpret_cast<unsigned char *>(vec + (3 + NROW) * mp) + ((mp + 15) & ~15));
}
__device__ __forceinline__ St carve_global(double *vec, double *L, int32_t *plist, int mp, Blk *bk, double *lds,
                                           int *slot_lds) {
  St s;
  s.mp = mp;
  s.bk = bk;
  s.lds = false;
  s.L = L;
  s.u = vec;
  s.g = vec + mp;
  s.dg = vec + 2 * mp;
  s.rows = vec + 3 * mp;
  s.x0 = lds ? lds : s.rows;
  s.yv = lds ? lds + mp : s.rows + 8 * mp;
  s.flag = reinterpret_cast<unsigned char *>(vec + (3 + NROW) * mp);
  s.plist = plist;
  s.slot = slot_lds;
  return s;
}
static_assert(kNnlsVecPerSlot == 3 + NROW + 1, "global NNLS state layout");

// ---- triangular solves ----------------------------------------------------

// Solves L X = R in place for the nr right-hand sides S.row(b)[k], k < n.
__device__ __forceinline__ void fwd_blk(const St &S, int n, int nr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int r0 = 0; r0 < n; r0 += TB) {
    const int e = n - r0 < TB ? n - r0 : TB;
    // diagonal block: wave w solves right-hand sides w, w + 4, w + 8; lane i holds row r0 + i
    if (wave < nr && lane < TB) {
      const int i = lane;
      const bool act = i < e;
      const int rb = act ? S.rowoff(r0 + i) + r0 : 0;
      double Lrow[TB];
      static_for<0, TB>([&](auto J) {
        constexpr int j = decltype(J)::value;
        Lrow[j] = (act && j < i) ? S.L[rb + j] : 0.0;
      });
      const double rd = act ? 1.0 / S.L[rb + i] : 0.0;
      double x[3];
      static_for<0, 3>([&](auto Qc) {
        constexpr int q = decltype(Qc)::value;
        const int b = wave + NW * q;
        x[q] = (act && b < nr) ? S.row(b)[r0 + i] : 0.0;
      });
      static_for<0, TB>([&](auto K) {
        constexpr int kk = decltype(K)::value;
        if (kk < e) {
          static_for<0, 3>([&](auto Qc) {
            constexpr int q = decltype(Qc)::value;
            if (wave + NW * q < nr) {
              const double xk = rl(x[q] * rd, kk);
              x[q] = i == kk ? xk : (i > kk ? fma(-Lrow[kk], xk, x[q]) : x[q]);
            }
          });
        }
      });
      static_for<0, 3>([&](auto Qc) {
        constexpr int q = decltype(Qc)::value;
        const int b = wave + NW * q;
        if (b < nr) {
          if (act) S.row(b)[r0 + i] = x[q];
          S.bk->xblk[b * TB + i] = x[q];
        }
      });
    }
    __syncthreads();
    if (r0 + TB < n) {
#if AMC_NNLS_NT > 256
      // rows below: r_row -= L[row, block] x_block, two rows per thread per
      // pass; every load of a pass (both rows of L, all right-hand sides) is
      // issued before the sums (the scratch rows all exist, so the loads of
      // right-hand sides past nr are harmless and unused)
      const double *xs = S.bk->xblk;
      for (int row = r0 + TB + tid; row < n; row += 2 * NT) {
        const int row2 = row + NT < n ? row + NT : row;
        const int rb = S.rowoff(row) + r0, rb2 = S.rowoff(row2) + r0;
        double La[TB], Lb[TB], xa[NRHS], xb2[NRHS];
        static_for<0, TB>([&](auto J) {
          constexpr int j = decltype(J)::value;
          La[j] = S.L[rb + j];
          Lb[j] = S.L[rb2 + j];
        });
        static_for<0, NRHS>([&](auto Bc) {
          constexpr int b = decltype(Bc)::value;
          xa[b] = S.row(b)[row];
          xb2[b] = S.row(b)[row2];
        });
        static_for<0, NRHS>([&](auto Bc) {
          constexpr int b = decltype(Bc)::value;
          if (b < nr) {
            double a0 = 0.0, a1 = 0.0, c0 = 0.0, c1 = 0.0;
            static_for<0, TB / 2>([&](auto J) {
              constexpr int j = decltype(J)::value;
              const double x0 = xs[b * TB + 2 * j], x1 = xs[b * TB + 2 * j + 1];
              a0 = fma(La[2 * j], x0, a0);
              a1 = fma(La[2 * j + 1], x1, a1);
              c0 = fma(Lb[2 * j], x0, c0);
              c1 = fma(Lb[2 * j + 1], x1, c1);
            });
            S.row(b)[row] = xa[b] - (a0 + a1);
            if (row2 != row) S.row(b)[row2] = xb2[b] - (c0 + c1);
          }
        });
      }
#else
      // rows below: r_row -= L[row, block] x_block
      const double *xs = S.bk->xblk;
      for (int row = r0 + TB + tid; row < n; row += NT) {
        const int rb = S.rowoff(row) + r0;
        double Lr[TB];
        static_for<0, TB>([&](auto J) {
          constexpr int j = decltype(J)::value;
          Lr[j] = S.L[rb + j];
        });
        for (int b = 0; b < nr; ++b) {
          double a0 = 0.0, a1 = 0.0;
          static_for<0, TB / 2>([&](auto J) {
            constexpr int j = decltype(J)::value;
            a0 = fma(Lr[2 * j], xs[b * TB + 2 * j], a0);
            a1 = fma(Lr[2 * j + 1], xs[b * TB + 2 * j + 1], a1);
          });
          S.row(b)[row] -= a0 + a1;
        }
      }
#endif
      __syncthreads();
    }
  }
}

// Solves L^T x = r in place for the vector x (factor order, length n >= 1).
__device__ __forceinline__ void bwd_blk(const St &S, int n, double *x) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int r0 = ((n - 1) / TB) * TB; r0 >= 0; r0 -= TB) {
    const int e = n - r0 < TB ? n - r0 : TB;
#if AMC_NNLS_NT > 256
    // the first pass of the column update reads no value the diagonal block
    // changes: its L loads are issued before the block is solved
    double pl[TB], pl2[TB];
    {
      const int c = tid < r0 ? tid : 0, c2 = tid + NT < r0 ? tid + NT : c;
      static_for<0, TB>([&](auto K) {
        constexpr int k = decltype(K)::value;
        const int rk = S.rowoff(k < e ? r0 + k : r0);
        pl[k] = S.L[rk + c];
        pl2[k] = S.L[rk + c2];
      });
    }
#endif
    if (wave == 0 && lane < TB) {
      const int i = lane;
      const bool act = i < e;
      double Lc[TB];  // column i of the diagonal block, rows below i
      static_for<0, TB>([&](auto K) {
        constexpr int kk = decltype(K)::value;
        Lc[kk] = (act && kk > i && kk < e) ? S.L[S.rowoff(r0 + kk) + r0 + i] : 0.0;
      });
      const double rd = act ? 1.0 / S.L[S.rowoff(act ? r0 + i : r0) + r0 + i] : 0.0;
      double xv = act ? x[r0 + i] : 0.0;
      static_for<0, TB>([&](auto K) {
        constexpr int kk = TB - 1 - decltype(K)::value;
        if (kk < e) {
          const double xk = rl(xv * rd, kk);
          xv = i == kk ? xk : (i < kk ? fma(-Lc[kk], xk, xv) : xv);
        }
      });
      if (act) x[r0 + i] = xv;
    }
    __syncthreads();
    // columns before the block: x_c -= sum_k L[r0 + k][c] x_{r0 + k}; the loads
    // of a column are all issued before the sums (rows past e read row r0)
#if AMC_NNLS_NT > 256
    for (int c = tid; c < r0; c += 2 * NT) {
      const int c2 = c + NT < r0 ? c + NT : c;
      double l[TB], l2[TB];
      if (c == tid) {
        static_for<0, TB>([&](auto K) {
          l[decltype(K)::value] = pl[decltype(K)::value];
          l2[decltype(K)::value] = pl2[decltype(K)::value];
        });
      } else {
        static_for<0, TB>([&](auto K) {
          constexpr int k = decltype(K)::value;
          const int rk = S.rowoff(k < e ? r0 + k : r0);
          l[k] = S.L[rk + c];
          l2[k] = S.L[rk + c2];
        });
      }
      const double xc = x[c], xc2 = x[c2];
      double a0 = 0.0, a1 = 0.0, b0 = 0.0, b1 = 0.0;
      static_for<0, TB / 2>([&](auto K) {
        constexpr int k = decltype(K)::value;
        if (2 * k < e) {
          a0 = fma(l[2 * k], x[r0 + 2 * k], a0);
          b0 = fma(l2[2 * k], x[r0 + 2 * k], b0);
        }
        if (2 * k + 1 < e) {
          a1 = fma(l[2 * k + 1], x[r0 + 2 * k + 1], a1);
          b1 = fma(l2[2 * k + 1], x[r0 + 2 * k + 1], b1);
        }
      });
      x[c] = xc - (a0 + a1);
      if (c2 != c) x[c2] = xc2 - (b0 + b1);
    }
#else
    for (int c = tid; c < r0; c += NT) {
      double l[TB];
      static_for<0, TB>([&](auto K) {
        constexpr int k = decltype(K)::value;
        l[k] = S.L[S.rowoff(k < e ? r0 + k : r0) + c];
      });
      double a0 = 0.0, a1 = 0.0;
      static_for<0, TB / 2>([&](auto K) {
        constexpr int k = decltype(K)::value;
        if (2 * k < e) a0 = fma(l[2 * k], x[r0 + 2 * k], a0);
        if (2 * k + 1 < e) a1 = fma(l[2 * k + 1], x[r0 + 2 * k + 1], a1);
      });
      x[c] -= a0 + a1;
    }
#endif
    __syncthreads();
  }
}

// ---- one-wave triangular solves (factor in LDS, n <= kWaveRows) ----------
//
// Column-oriented substitution in a single wave, with no block barriers: lane
// l holds rows l, l + 64 and l + 128; once x_k is known (r_k / L_kk, read
// from its lane) it is applied to the rows still open.  Every update is a
// plain fma with a zero coefficient where a row is not touched, so the lanes
// run without branches.  The substitution is the same sequence of
// operations as the blocked solves, one product at a time.

constexpr int kWaveRows = 192;

// Columns in flight ahead of the one being applied: the LDS latency spans a
// few substitution steps.  The empty asm with a memory clobber after each
// step's loads keeps the compiler from folding the loop-carried loads back
// into one load per step at the point of use.
constexpr int kPD = 4;

// L X = R for the nr right-hand sides S.row(b), b < nr, in place: wave w
// takes right-hand sides w, w + NW and w + 2 NW.  Column k of L, below row k,
// is read from the packed rows (L[tri(i) + k]).
__device__ __forceinline__ void fwd_wave(const St &S, int n, int nr) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < nr) {
    int rbase[3];
    double rd[3], xv[3][3];
    static_for<0, 3>([&](auto Mc) {
      constexpr int m = decltype(Mc)::value;
      const int i = lane + 64 * m;
      rbase[m] = i < n ? tri(i) : 0;  // rows past n read row 0's area (the value is not used)
      rd[m] = i < n ? 1.0 / S.L[rbase[m] + i] : 0.0;
      static_for<0, 3>([&](auto Qc) {
        constexpr int q = decltype(Qc)::value;
        const int b = wave + NW * q;
        xv[q][m] = (b < nr && i < n) ? S.row(b)[i] : 0.0;
      });
    });
    static_for<0, 3>([&](auto Mc) {
      constexpr int M = decltype(Mc)::value;
      const int k0 = 64 * M, k1 = n < 64 * M + 64 ? n : 64 * M + 64;
      if (k0 < k1) {
        double ring[kPD][3];
        static_for<0, kPD>([&](auto Pc) {
          constexpr int j = decltype(Pc)::value;
          const int kc = k0 + j < k1 ? k0 + j : k1 - 1;
          static_for<0, 3>([&](auto Rc) {
            constexpr int m = decltype(Rc)::value;
            ring[j][m] = m >= M ? S.L[rbase[m] + kc] : 0.0;
          });
        });
        // step k applies column k, held in ring slot k % kPD, then refills the
        // slot with column k + kPD (full trips of kPD steps; the last few steps
        // take no refill, so no step is conditional inside a trip)
        auto step = [&](int k, double(&slot)[3], auto refill) __attribute__((always_inline)) {
          const int kl = k - 64 * M;
          double lc[3];
          static_for<M, 3>([&](auto Rc) {
            constexpr int m = decltype(Rc)::value;
            lc[m] = ((m > M || lane > kl) && lane + 64 * m < n) ? slot[m] : 0.0;
          });
          if constexpr (decltype(refill)::value) {
            const int kn = k + kPD < k1 ? k + kPD : k1 - 1;
            static_for<M, 3>([&](auto Rc) {
              constexpr int m = decltype(Rc)::value;
              slot[m] = S.L[rbase[m] + kn];
            });
            asm volatile("" ::: "memory");
          }
          static_for<0, 3>([&](auto Qc) {
            constexpr int q = decltype(Qc)::value;
            if (wave + NW * q < nr) {
              const double xk = rl(xv[q][M] * rd[M], kl);
              static_for<M, 3>([&](auto Rc) {
                constexpr int m = decltype(Rc)::value;
                xv[q][m] = fma(-lc[m], xk, xv[q][m]);
              });
            }
          });
        };
        int k = k0;
        for (; k + kPD <= k1; k += kPD)
          static_for<0, kPD>([&](auto Pc) { step(k + decltype(Pc)::value, ring[decltype(Pc)::value], std::true_type{}); });
        static_for<0, kPD - 1>([&](auto Pc) {
          constexpr int j = decltype(Pc)::value;
          if (k + j < k1) step(k + j, ring[j], std::false_type{});
        });
      }
    });
    static_for<0, 3>([&](auto Mc) {
      constexpr int m = decltype(Mc)::value;
      const int i = lane + 64 * m;
      static_for<0, 3>([&](auto Qc) {
        constexpr int q = decltype(Qc)::value;
        const int b = wave + NW * q;
        if (b < nr && i < n) S.row(b)[i] = xv[q][m] * rd[m];
      });
    });
  }
  __syncthreads();
}

// L^T x = r in place for the vector x, in wave 0.  Column k of L^T is row k
// of L, contiguous in the packed factor.
__device__ __forceinline__ void bwd_wave(const St &S, int n, double *x) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    double rd[3], xv[3];
    static_for<0, 3>([&](auto Mc) {
      constexpr int m = decltype(Mc)::value;
      const int i = lane + 64 * m;
      rd[m] = i < n ? 1.0 / S.L[tri(i) + i] : 0.0;
      xv[m] = i < n ? x[i] : 0.0;
    });
    static_for<0, 3>([&](auto Mc) {
      constexpr int M = 2 - decltype(Mc)::value;
      const int kt = 64 * M, k1 = (n < 64 * M + 64 ? n : 64 * M + 64) - 1;
      if (k1 >= kt) {
        // row k of L at the lanes' columns (columns at or past k read the
        // row's first entry; the value is not used)
        auto load_row = [&](int k, double(&slot)[3]) __attribute__((always_inline)) {
          static_for<0, M + 1>([&](auto Rc) {
            constexpr int m = decltype(Rc)::value;
            slot[m] = S.L[tri(k) + (m < M || lane < k - kt ? lane + 64 * m : 0)];
          });
        };
        double ring[kPD][3];
        static_for<0, kPD>([&](auto Pc) {
          constexpr int j = decltype(Pc)::value;
          load_row(k1 - j >= kt ? k1 - j : kt, ring[j]);
        });
        auto step = [&](int k, double(&slot)[3], auto refill) __attribute__((always_inline)) {
          const int kl = k - kt;
          double use[3];
          static_for<0, M + 1>([&](auto Rc) {
            constexpr int m = decltype(Rc)::value;
            use[m] = slot[m];
          });
          if constexpr (decltype(refill)::value) {
            load_row(k - kPD >= kt ? k - kPD : kt, slot);
            asm volatile("" ::: "memory");
          }
          const double xk = rl(xv[M] * rd[M], kl);
          static_for<0, M>([&](auto Rc) {
            constexpr int m = decltype(Rc)::value;
            xv[m] = fma(-use[m], xk, xv[m]);
          });
          const double l = lane < kl ? use[M] : 0.0;
          xv[M] = fma(-l, xk, xv[M]);
        };
        int k = k1;
        for (; k - (kPD - 1) >= kt; k -= kPD)
          static_for<0, kPD>([&](auto Pc) { step(k - decltype(Pc)::value, ring[decltype(Pc)::value], std::true_type{}); });
        static_for<0, kPD - 1>([&](auto Pc) {
          constexpr int j = decltype(Pc)::value;
          if (k - j >= kt) step(k - j, ring[j], std::false_type{});
        });
      }
    });
    static_for<0, 3>([&](auto Mc) {
      constexpr int m = decltype(Mc)::value;
      const int i = lane + 64 * m;
      if (i < n) x[i] = xv[m] * rd[m];
    });
  }
  __syncthreads();
}

// Forward and backward solves: one wave when the factor is in LDS and small
// enough, else the blocked form.
__device__ __forceinline__ void fwd_solve(const St &S, int n, int nr) {
  if (S.lds && n <= kWaveRows)
    fwd_wave(S, n, nr);
  else
    fwd_blk(S, n, nr);
}
__device__ __forceinline__ void bwd_solve(const St &S, int n, double *x) {
  if (S.lds && n <= kWaveRows)
    bwd_wave(S, n, x);
  else
    bwd_blk(S, n, x);
}

// ---- gradient of the zero variables ---------------------------------------

// u_snap = u, g_snap = g (rows 9 and 10)
__device__ __forceinline__ void snapshot(const St &S, int p) {
  double *us = S.rows + 9 * S.mp, *gs = S.rows + 10 * S.mp;
  for (int a = threadIdx.x; a < p; a += NT) {
    us[a] = S.u[a];
    gs[a] = S.g[a];
  }
  __syncthreads();
}

// Brings g up to date on every zero variable by the exact increment since the
// last snapshot, g_a = g_a(snap) - Gs_a (u - u_snap), then takes a new
// snapshot of u and g.  Only the zero variables (neither free nor blocked)
// need it, and G is symmetric, so each takes one row of G: row a dotted with
// the scaled change (row 2, dense: (u - u_snap) / dg, zero where unchanged).
// When few variables changed, the row is read at the changed positions only
// (row 1: their indices, in increasing order, and their scaled change packed
// in row 3).  One wave per zero variable (list in row 4), lanes over the row
// in a fixed order, so the result does not depend on timing.  Where the
// solve vector lives apart from the scratch rows (in LDS), the dense change
// takes its place: every wave reads it once per zero variable, and the solve
// vector holds nothing between a settle and the next block entry.
__device__ __forceinline__ void sync_z(const St &S, const double *G, int64_t ld, int p) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mp = S.mp;
  Blk *bk = S.bk;
  int *lst = reinterpret_cast<int *>(S.rows + mp);
  double *dv = S.x0 != S.rows ? S.x0 : S.rows + 2 * mp;
  double *dvc = S.rows + 3 * mp;
  int *zl = reinterpret_cast<int *>(S.rows + 4 * mp);
  const double *us = S.rows + 9 * mp;
  double *gs = S.rows + 10 * mp;
  int ns = 0, nz = 0;
  for (int c0 = 0; c0 < p; c0 += NT) {
    const int c = c0 + tid;
    double dl = 0.0;
    bool zero = false;
    if (c < p) {
      dl = (S.u[c] - us[c]) / S.dg[c];
      dv[c] = dl;
      zero = !(S.flag[c] & (F_PASSIVE | F_BLOCKED));
    }
    const bool pred = dl != 0.0;
    const unsigned long long bal = __ballot(pred);
    const unsigned long long balz = __ballot(zero);
    if (lane == 0) bk->wc[wave] = __popcll(bal);
    __syncthreads();
    int off = ns;
    for (int v = 0; v < wave; ++v) off += bk->wc[v];
    if (pred) {
      const int at = off + __popcll(bal & ((1ull << lane) - 1ull));
      lst[at] = c;
      dvc[at] = dl;
    }
    for (int v = 0; v < NW; ++v) ns += bk->wc[v];
    __syncthreads();
    if (lane == 0) bk->wc[wave] = __popcll(balz);
    __syncthreads();
    int offz = nz;
    for (int v = 0; v < wave; ++v) offz += bk->wc[v];
    if (zero) zl[offz + __popcll(balz & ((1ull << lane) - 1ull))] = c;
    for (int v = 0; v < NW; ++v) nz += bk->wc[v];
    __syncthreads();
  }
  if (ns > 0) {
    const bool sparse = ns * 8 < p;
    for (int k = wave; k < nz; k += NW) {
      const int a = zl[k];
      const double *Ga = G + int64_t(a) * ld;
      double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
      if (sparse) {
        for (int k2 = lane; k2 < ns; k2 += 64) acc[0] = fma(Ga[lst[k2]], dvc[k2], acc[0]);
      } else {
        int c0 = 0;
        for (; c0 + 512 <= p; c0 += 512) {
          double v[8];
          static_for<0, 8>([&](auto U) {
            constexpr int u = decltype(U)::value;
            v[u] = Ga[c0 + 64 * u + lane];
          });
          static_for<0, 8>([&](auto U) {
            constexpr int u = decltype(U)::value;
            acc[u] = fma(v[u], dv[c0 + 64 * u + lane], acc[u]);
          });
        }
        for (int c = c0 + lane; c < p; c += 64) acc[0] = fma(Ga[c], dv[c], acc[0]);
      }
      const double z = wave_sum(((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7])));
      if (lane == 0) S.g[a] = gs[a] - z / S.dg[a];
    }
  } else {
    for (int k = tid; k < nz; k += NT) S.g[zl[k]] = gs[zl[k]];
  }
  __syncthreads();
  snapshot(S, p);
}

// ---- factor updates --------------------------------------------------------

// row of packed lower-triangle index s
__device__ __forceinline__ int row_of(int s) {
  int i = int((sqrtf(8.0f * float(s) + 1.0f) - 1.0f) * 0.5f);
  if (tri(i + 1) <= s) ++i;
  if (tri(i) > s) --i;
  return i;
}

// Deletes factor position q: rows below move up one position without column
// q, then the trailing rows absorb the removed column by a rank-one update
// (Givens rotations, applied 16 columns at a time).  y = L^-1 g_P follows:
// its entries below q take the same rotations, with y_q as the extra entry.
// Packed rows move in memory; slotted rows (kSlotRows) stay in their slots,
// the removed row's slot goes to the free end of the slot list, and the
// rotation pass reads each row's columns past q one place to the right of
// where it writes them.
__device__ __forceinline__ void remove_at(const St &S, int q) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Blk *bk = S.bk;
  const int np = bk->np, n2 = np - 1;
  double *xc = S.rows + 7 * S.mp;
  double *yv = S.yv;
  double z = yv[q];  // y of the removed position, rotated into the trailing entries below
  const int freed = kSlotRows ? S.slot[q] : 0;
  if constexpr (!kSlotRows)
    for (int i = q + 1 + tid; i < np; i += NT) xc[i - 1] = S.L[tri(i) + q];
  // Every element moves to a lower index, so chunks taken in increasing
  // source order never overwrite a source that is still to be read.
  for (int base = q; base < n2; base += NT) {
    const int k = base + tid;
    const int pv = k < n2 ? S.plist[k + 1] : 0;
    const double yk = k < n2 ? yv[k + 1] : 0.0;
    int sv = 0;
    if constexpr (kSlotRows) sv = k < n2 ? S.slot[k + 1] : 0;
    __syncthreads();
    if (k < n2) {
      S.plist[k] = pv;
      yv[k] = yk;
      if constexpr (kSlotRows) S.slot[k] = sv;
    }
  }
  if constexpr (kSlotRows) {
    if (tid == 0) S.slot[n2] = freed;
    __syncthreads();
    for (int k = q + tid; k < n2; k += NT) xc[k] = S.L[S.rowoff(k) + q];
  } else {
  const int s0 = tri(q + 1), s1 = tri(np);
  for (int base = s0; base < s1; base += NT * 16) {
    double v[16];
    int dst[16];
    static_for<0, 16>([&](auto U) {
      constexpr int u = decltype(U)::value;
      const int s = base + u * NT + tid;
      dst[u] = -1;
      v[u] = 0.0;
      if (s < s1) {
        const int i = row_of(s);
        const int c = s - tri(i);
        if (c != q) {
          dst[u] = tri(i - 1) + (c < q ? c : c - 1);
          v[u] = S.L[s];
        }
      }
    });
    __syncthreads();
    static_for<0, 16>([&](auto U) {
      constexpr int u = decltype(U)::value;
      if (dst[u] >= 0) S.L[dst[u]] = v[u];
    });
  }
  }
  __syncthreads();
  // rank-one update: L' L'^T = L L^T + x x^T on positions q..n2-1
  constexpr int sh = kSlotRows ? 1 : 0;  // column offset of a row's unrotated entries past q
  if (!kSlotRows && S.lds && n2 <= kWaveRows) {
    // in wave 0: rotation k comes from (L_kk, x_k), read from lane k's
    // registers, and turns column k of every row below it at once
    if (wave == 0) {
      int rbase[3];
      double xv[3], yl[3];
      static_for<0, 3>([&](auto Mc) {
        constexpr int m = decltype(Mc)::value;
        const int i = lane + 64 * m;
        const bool act = i >= q && i < n2;
        rbase[m] = act ? tri(i) : 0;
        xv[m] = act ? xc[i] : 0.0;
        yl[m] = act ? yv[i] : 0.0;
      });
      // (columns and diagonals kPD steps ahead are loaded before a step's
      // rotation; a step writes only its own column and diagonal)
      static_for<0, 3>([&](auto Mc) {
        constexpr int M = decltype(Mc)::value;
        const int kb = q > 64 * M ? q : 64 * M, k1 = n2 < 64 * M + 64 ? n2 : 64 * M + 64;
        if (kb < k1) {
          double ring[kPD][4];  // column k at the lane's rows m >= M, then L_kk
          auto load_col = [&](int k, double(&sl)[4]) __attribute__((always_inline)) {
            static_for<M, 3>([&](auto Rc) {
              constexpr int m = decltype(Rc)::value;
              sl[m] = S.L[rbase[m] + k];
            });
            sl[3] = S.L[tri(k) + k];
          };
          static_for<0, kPD>([&](auto Pc) {
            constexpr int j = decltype(Pc)::value;
            load_col(kb + j < k1 ? kb + j : k1 - 1, ring[j]);
          });
          auto step = [&](int k, double(&sl)[4], auto refill) __attribute__((always_inline)) {
            double use[4];
            static_for<0, 4>([&](auto Uc) { use[decltype(Uc)::value] = sl[decltype(Uc)::value]; });
            if constexpr (decltype(refill)::value) {
              load_col(k + kPD < k1 ? k + kPD : k1 - 1, sl);
              asm volatile("" ::: "memory");
            }
            const int kl = k - 64 * M;
            const int dk = tri(k) + k;
            const double lkk = use[3];
            const double xk = rl(xv[M], kl);
            const double t2 = fma(lkk, lkk, xk * xk);
            const double ri = rsqrt(t2);
            const double c = lkk * ri, s = xk * ri;
            const double yk = rl(yl[M], kl);
            if (lane == kl) {
              yl[M] = fma(c, yk, s * z);
              S.L[dk] = t2 * ri;
            }
            z = fma(c, z, -s * yk);
            static_for<M, 3>([&](auto Rc) {
              constexpr int m = decltype(Rc)::value;
              if ((m > M || lane > kl) && lane + 64 * m < n2) {
                const double l = use[m];
                S.L[rbase[m] + k] = fma(c, l, s * xv[m]);
                xv[m] = fma(c, xv[m], -s * l);
              }
            });
          };
          int k = kb;
          for (; k + kPD <= k1; k += kPD)
            static_for<0, kPD>([&](auto Pc) { step(k + decltype(Pc)::value, ring[decltype(Pc)::value], std::true_type{}); });
          static_for<0, kPD - 1>([&](auto Pc) {
            constexpr int j = decltype(Pc)::value;
            if (k + j < k1) step(k + j, ring[j], std::false_type{});
          });
        }
      });
      static_for<0, 3>([&](auto Mc) {
        constexpr int m = decltype(Mc)::value;
        const int i = lane + 64 * m;
        if (i >= q && i < n2) yv[i] = yl[m];
      });
    }
    __syncthreads();
  } else
  for (int k0 = q; k0 < n2; k0 += TB) {
    const int e = n2 - k0 < TB ? n2 - k0 : TB;
    if (wave == 0 && lane < TB) {
      const int i = lane;
      const bool act = i < e;
      const int rb = act ? S.rowoff(k0 + i) + k0 : 0;
      double Lr[TB];
      static_for<0, TB>([&](auto J) {
        constexpr int j = decltype(J)::value;
        Lr[j] = (act && j <= i) ? S.L[rb + j + sh] : 0.0;
      });
      double xv = act ? xc[k0 + i] : 0.0;
      double yl = act ? yv[k0 + i] : 0.0;
      static_for<0, TB>([&](auto K) {
        constexpr int kk = decltype(K)::value;
        if (kk < e) {
          const double lkk = rl(Lr[kk], kk), xk = rl(xv, kk);
          const double t2 = fma(lkk, lkk, xk * xk);
          const double ri = rsqrt(t2);
          const double c = lkk * ri, s = xk * ri;
          const double yk = rl(yl, kk);
          if (i == kk) yl = fma(c, yk, s * z);
          z = fma(c, z, -s * yk);
          if (i == kk) {
            Lr[kk] = t2 * ri;
          } else if (i > kk) {
            const double l = Lr[kk];
            Lr[kk] = fma(c, l, s * xv);
            xv = fma(c, xv, -s * l);
          }
          if (lane == 0) {
            bk->cs[2 * kk] = c;
            bk->cs[2 * kk + 1] = s;
          }
        }
      });
      if (act) {
        static_for<0, TB>([&](auto J) {
          constexpr int j = decltype(J)::value;
          if (j <= i) S.L[rb + j] = Lr[j];
        });
        yv[k0 + i] = yl;
      }
    }
    __syncthreads();
    if (k0 + TB < n2) {
      for (int row = k0 + TB + tid; row < n2; row += NT) {
        const int rb = S.rowoff(row) + k0;
        double Lr[TB];
        static_for<0, TB>([&](auto J) {
          constexpr int j = decltype(J)::value;
          Lr[j] = S.L[rb + j + sh];
        });
        double xv = xc[row];
        static_for<0, TB>([&](auto K) {
          constexpr int kk = decltype(K)::value;
          const double c = bk->cs[2 * kk], s = bk->cs[2 * kk + 1];
          const double l = Lr[kk];
          Lr[kk] = fma(c, l, s * xv);
          xv = fma(c, xv, -s * l);
        });
        static_for<0, TB>([&](auto J) {
          constexpr int j = decltype(J)::value;
          S.L[rb + j] = Lr[j];
        });
        xc[row] = xv;
      }
      __syncthreads();
    }
  }
  if (tid == 0) bk->np = n2;
  __syncthreads();
}

// Largest factor position k < np with pred(k) true, -1 if none.
template <typename P>
__device__ __forceinline__ int last_position(int np, P pred, Red *red) {
  int best = -1;
  for (int k = threadIdx.x; k < np; k += NT)
    if (pred(k)) best = k;
  double v;
  return block_argmax(double(best), best, red, &v);
}

// Appends the nc <= NB candidates in bk->cand (zero, not blocked) to the free
// set.  One blocked forward pass over the current factor gives each
// candidate's row l = L^-1 Gs[P, j] and y = L^-1 g_P; a Cholesky of the block
// finishes the rows (candidates whose pivot vanishes are blocked).  On return
// x0 holds y = L^-1 g_P over the extended free set and bk->ctl[2] the number
// of accepted candidates.  Rows 1..8 are overwritten.
__device__ __forceinline__ void block_append(const St &S, const double *G, int64_t ld, int nc, int *status) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Blk *bk = S.bk;
  const int np0 = bk->np;
  for (int k = tid; k < np0; k += NT) {
    const int a = S.plist[k];
    const double da = S.dg[a];
    S.x0[k] = S.g[a];
    // the NB loads of a position are issued together (slots past nc read
    // the first candidate's row and are not stored)
    double gv[NB];
    static_for<0, NB>([&](auto Bc) {
      constexpr int b = decltype(Bc)::value;
      gv[b] = G[int64_t(bk->cand[b < nc ? b : 0]) * ld + a];
    });
    static_for<0, NB>([&](auto Bc) {
      constexpr int b = decltype(Bc)::value;
      if (b < nc) S.row(b + 1)[k] = gv[b] / (S.dg[bk->cand[b]] * da);
    });
  }
  if (tid < nc * nc) {
    const int j1 = bk->cand[tid / nc], j2 = bk->cand[tid % nc];
    bk->Gc[(tid / nc) * NB + tid % nc] = G[int64_t(j1) * ld + j2] / (S.dg[j1] * S.dg[j2]);
  }
  __syncthreads();
  if (np0 > 0) fwd_solve(S, np0, nc + 1);
  // dots[b1][b2] = <rhs_b1, rhs_b2> over the old positions, b2 <= b1 (one wave per pair)
  const int npair = (nc + 1) * (nc + 2) / 2;
  for (int pr = wave; pr < npair; pr += NW) {
    int b1 = 0;
    while ((b1 + 1) * (b1 + 2) / 2 <= pr) ++b1;
    const int b2 = pr - b1 * (b1 + 1) / 2;
    const double *r1 = S.row(b1), *r2 = S.row(b2);
    double v = 0.0;
    for (int k = lane; k < np0; k += 64) v = fma(r1[k], r2[k], v);
    v = wave_sum(v);
    if (lane == 0) bk->dots[b1 * NRHS + b2] = v;
  }
  __syncthreads();
  // Cholesky of the candidate block in wave 0 (wave-uniform values in registers)
  if (wave == 0) {
    double E[NB][NB], Dg[NB], yb[NB];
    int idx[NB];
    int nacc = 0;
    static_for<0, NB>([&](auto A) {
      constexpr int a = decltype(A)::value;
      Dg[a] = 1.0;
      yb[a] = 0.0;
      idx[a] = 0;
      static_for<0, NB>([&](auto A2) { E[a][decltype(A2)::value] = 0.0; });
    });
    static_for<0, NB>([&](auto Bc) {
      constexpr int b = decltype(Bc)::value;
      if (b < nc) {
        const int j = bk->cand[b];
        double row[NB];
        double ss = bk->dots[(b + 1) * NRHS + (b + 1)];
        double yy = S.g[j] - bk->dots[(b + 1) * NRHS];
        static_for<0, NB>([&](auto A) {
          constexpr int a = decltype(A)::value;
          row[a] = 0.0;
          if (a < nacc) {
            const int bb = idx[a];
            double v = bk->Gc[b * NB + bb] - bk->dots[(b + 1) * NRHS + (bb + 1)];
            static_for<0, a>([&](auto A2) {
              constexpr int a2 = decltype(A2)::value;
              v -= row[a2] * E[a][a2];
            });
            v /= Dg[a];
            row[a] = v;
            ss += v * v;
            yy -= v * yb[a];
          }
        });
        const double d2 = bk->Gc[b * NB + b] - ss;
        if (d2 > PIV_TOL) {
          const double dd = sqrt(d2);
          static_for<0, NB>([&](auto A) {
            constexpr int a = decltype(A)::value;
            if (a == nacc) {
              static_for<0, a>([&](auto A2) {
                constexpr int a2 = decltype(A2)::value;
                E[a][a2] = row[a2];
              });
              Dg[a] = dd;
              yb[a] = yy / dd;
              idx[a] = b;
            }
          });
          ++nacc;
        } else if (lane == 0) {
          S.flag[j] = F_BLOCKED;
          *status |= int(AMC_HS_NNLS_SINGULAR);
        }
      }
    });
    if (lane == 0) {
      static_for<0, NB>([&](auto A) {
        constexpr int a = decltype(A)::value;
        bk->Dg[a] = Dg[a];
        bk->yb[a] = yb[a];
        bk->accb[a] = idx[a];
        static_for<0, a>([&](auto A2) {
          constexpr int a2 = decltype(A2)::value;
          bk->E[a * NB + a2] = E[a][a2];
        });
      });
      bk->ctl[2] = nacc;
    }
  }
  __syncthreads();
  const int nacc = bk->ctl[2];
  for (int a = 0; a < nacc; ++a) {
    const int b = bk->accb[a];
    const int pos = np0 + a;
    const int base = S.rowoff(pos);
    const double *rb = S.row(b + 1);
    for (int k = tid; k < np0; k += NT) S.L[base + k] = rb[k];
    if (tid < a) S.L[base + np0 + tid] = bk->E[a * NB + tid];
    if (tid == 0) {
      const int j = bk->cand[b];
      S.L[base + pos] = bk->Dg[a];
      S.plist[pos] = j;
      S.flag[j] = F_PASSIVE | F_NEW;
      S.x0[pos] = bk->yb[a];
    }
  }
  __syncthreads();
  if (tid == 0) bk->np = np0 + nacc;
  __syncthreads();
}

// Least squares on the free set, with feasibility back-tracking, starting
// from a feasible u whose support is the free set; variables that just
// entered sit at zero, flagged F_NEW.  have_y: x0 holds y = L^-1 g_P.
//  - An entering variable whose solution is not positive leaves again before
//    any step is taken.  If it entered alone it is set aside for the rest of
//    this fit (Lawson and Hanson's guard against cycling on round-off);
//    otherwise later blocks of candidates are half as large (ctl[3]; one at
//    a time once it reaches 1).  In the workspace-resident build (large
//    budgets) a block none of whose variables leaves this way doubles the
//    size again, up to NB (ctl[6] records a drop), so that a refit with many
//    new keys does not take the rest of them one by one.
//  - Otherwise the iterate moves toward the solution, as far as feasibility
//    allows, and the variables that reach zero leave.
// Only the free-set rows of g change here (by the factor's model); y follows
// every step and every removal.
__device__ __forceinline__ void settle(const St &S, int p, bool have_y, bool single, Red *red) {
  const int tid = threadIdx.x;
  Blk *bk = S.bk;
  __syncthreads();
  if (bk->np == 0) return;
  if (!have_y) {
    for (int k = tid; k < bk->np; k += NT) S.x0[k] = S.g[S.plist[k]];
    __syncthreads();
    fwd_solve(S, bk->np, 1);
  }
  for (int k = tid; k < bk->np; k += NT) S.yv[k] = S.x0[k];
  for (int guard = 0; guard < 4 * S.mp + 8; ++guard) {
    __syncthreads();
    const int np = bk->np;
    if (np == 0) break;
    for (int k = tid; k < np; k += NT) S.x0[k] = S.yv[k];
    __syncthreads();
    bwd_solve(S, np, S.x0);  // x0 = Gs_PP^-1 g_P: the step to the free-set optimum
    int ndrop = 0;
    double best = INFINITY;
    int kb = -1;
    for (int k = tid; k < np; k += NT) {
      const int a = S.plist[k];
      const double d = S.x0[k];
      const double ua = S.u[a];
      if ((S.flag[a] & F_NEW) && ua == 0.0 && !(d > 0.0)) {
        S.flag[a] |= F_DROP;
        ++ndrop;
      } else if (ua + d <= 0.0) {
        const double rt = d < 0.0 ? ua / (-d) : 0.0;
        if (kb < 0 || rt < best) {
          best = rt;
          kb = k;
        }
      }
    }
    ndrop = block_count(ndrop, red);
    if (ndrop > 0) {
      for (;;) {
        const int q = last_position(bk->np, [&](int k) { return (S.flag[S.plist[k]] & F_DROP) != 0; }, red);
        if (q < 0) break;
        if (tid == 0) {
          S.flag[S.plist[q]] = single ? F_BLOCKED : 0;
          if (!single) bk->ctl[3] = bk->ctl[5] > 1 ? bk->ctl[5] / 2 : 1;
          bk->ctl[6] = 1;
        }
        __syncthreads();
        remove_at(S, q);
      }
      continue;
    }
    double nbest;
    kb = block_argmax(kb >= 0 ? -best : -INFINITY, kb, red, &nbest);
    best = -nbest;
    const bool done = kb < 0;
    const double alpha = done ? 1.0 : (best < 1.0 ? best : 1.0);
    const double keep = done ? 0.0 : 1.0 - alpha;
    for (int k = tid; k < np; k += NT) {
      const int a = S.plist[k];
      const double ua = S.u[a];
      const double d = S.x0[k];
      const double un = done ? ua + d : ((k == kb) ? 0.0 : fma(alpha, d, ua));
      S.u[a] = un > 0.0 ? un : 0.0;
      S.flag[a] &= ~F_NEW;
      S.g[a] *= keep;
      S.yv[k] *= keep;
    }
    __syncthreads();
    if (done) break;
    // every free variable that reached zero leaves (highest position first)
    for (;;) {
      const int q = last_position(bk->np, [&](int k) { return !(S.u[S.plist[k]] > 0.0); }, red);
      if (q < 0) break;
      if (tid == 0) {
        const int a = S.plist[q];
        S.u[a] = 0.0;
        S.flag[a] &= ~(F_PASSIVE | F_NEW);
      }
      __syncthreads();
      remove_at(S, q);
    }
  }
  __syncthreads();
}

// Up to maxc zero variables with the largest gradients above tol (ties to the
// lower index) go to bk->cand; returns their count.
__device__ __forceinline__ int pick_candidates(const St &S, int p, double tol, int maxc, Red *red) {
  int nc = 0;
  for (; nc < maxc; ++nc) {
    double bv = -INFINITY;
    int bi = -1;
    for (int a = threadIdx.x; a < p; a += NT) {
      if (!(S.flag[a] & (F_PASSIVE | F_BLOCKED | F_CAND))) {
        const double v = S.g[a];
        if (v > tol && (bi < 0 || v > bv)) {
          bv = v;
          bi = a;
        }
      }
    }
    double v;
    bi = block_argmax(bv, bi, red, &v);
    if (bi < 0) break;
    if (threadIdx.x == 0) {
      S.bk->cand[nc] = bi;
      S.flag[bi] |= F_CAND;
    }
    __syncthreads();
  }
  return nc;
}

// One block solves one system on the state S (u, g, dg, flag set up by
// nnls_setup for a < p; L, plist and bk->np hold the starting free set).
//   tol, cap : KKT tolerance on the scaled gradient and outer-iteration cap
//   support  : the positive entries of u enter the free set first (warm
//              start of the stand-alone solver)
__device__ __forceinline__ void nnls_core(const St &S, const double *G, int64_t ld, int p, double tol, int cap,
                                          bool support, Red *red, int *status, int *iters_out) {
  const int tid = threadIdx.x;
  Blk *bk = S.bk;
  int iters = 0;
  if (support) {
    // the support of the warm start becomes the free set, NB variables at a time
    int a0 = 0;
    for (;;) {
      __syncthreads();
      if (tid == 0) {
        int nc = 0;
        for (; a0 < p && nc < NB; ++a0)
          if (S.u[a0] > 0.0 && !(S.flag[a0] & (F_PASSIVE | F_BLOCKED))) bk->cand[nc++] = a0;
        bk->ctl[1] = nc;
        bk->ctl[4] = a0;
      }
      __syncthreads();
      const int nc = bk->ctl[1];
      a0 = bk->ctl[4];
      if (nc == 0) break;
      block_append(S, G, ld, nc, status);
    }
    for (int k = tid; k < bk->np; k += NT) S.flag[S.plist[k]] &= ~F_NEW;
    // a dependent variable dropped here still carries weight: take it out of u and g
    double *tmp = S.rows + 2 * S.mp;
    for (int a = tid; a < p; a += NT) tmp[a] = ((S.flag[a] & F_BLOCKED) && S.u[a] > 0.0) ? -S.u[a] : 0.0;
    __syncthreads();
    for (int a = tid; a < p; a += NT) {
      double acc = 0.0;
      for (int c = 0; c < p; ++c)
        if (tmp[c] != 0.0) acc = fma(G[int64_t(c) * ld + a], tmp[c] / S.dg[c], acc);
      S.g[a] -= acc / S.dg[a];
    }
    __syncthreads();
    for (int a = tid; a < p; a += NT)
      if (S.flag[a] & F_BLOCKED) S.u[a] = 0.0;
    __syncthreads();
    snapshot(S, p);
  }
  // refine the starting free set with the gradient given
  settle(S, p, false, false, red);
  for (;;) {
    sync_z(S, G, ld, p);
    const int nc = pick_candidates(S, p, tol, bk->ctl[3], red);
    if (nc == 0) break;
    if (iters >= cap) {
      if (tid == 0) *status |= int(AMC_HS_NNLS_CAP);
      break;
    }
    ++iters;
    if (tid == 0) {
      bk->ctl[5] = nc;
      bk->ctl[6] = 0;
    }
    block_append(S, G, ld, nc, status);
    if (bk->ctl[2] > 0) settle(S, p, true, nc == 1, red);
    if (kGrowBlocks && tid == 0 && bk->ctl[6] == 0 && bk->ctl[2] == nc)
      bk->ctl[3] = bk->ctl[3] < NB / 2 ? 2 * bk->ctl[3] : NB;
  }
  __syncthreads();
  *iters_out = iters;
}

// Entering tolerances relative to max |b| in unit-diagonal form (when the
// caller gives none).  The refits that steer the selection on the Gram form
// take the textbook worst case of the gradient's rounding, 10 eps p.  The
// final refit, whose weights are the output, the refits that warm-start the
// exact refit, and the stand-alone solver take half an ulp of the largest
// |b|: any gradient the float64 data resolve.  Once the mass is fitted
// to a small residual the true gradients of keys that the minimiser still
// needs fall below 10 eps p (a 2048-key head ended with beta off by 0.11, a
// 700-key one by 6); a variable entered on a gradient at rounding level whose
// solution is not positive leaves again and is set aside for the rest of the
// fit.  Heads above kNnlsFineMaxT keys keep the coarse test in the polish too:
// with the fine one a single 6000-key head's polish ran past three minutes
// (each active-set step there walks a factor of up to 6000 rows in global
// memory), and the fine test in every refit would cost more still.
__device__ __forceinline__ double nnls_tol_coarse(int p) { return 10.0 * DBL_EPSILON * double(p); }
constexpr double kNnlsTolFine = 0.5 * DBL_EPSILON;
constexpr int64_t kNnlsFineMaxT = 2048;

// Sets up u, g, dg, flag for a < p from G, b, the warm start (first nwarm
// entries of w) and the accurate gradient gA (nullable: formed from G and
// b), and marks the starting free set.  Returns the KKT tolerance, 0 when
// there is nothing to fit (auto_tol: the entering test when prm gives none).
__device__ __forceinline__ double nnls_setup(const St &S, const double *G, int64_t ld, int p, const double *b,
                                             const double *gA, const double *w, int nwarm, const NnlsParams &prm,
                                             double auto_tol, Red *red) {
  const int tid = threadIdx.x;
  double bl = 0.0;
  for (int a = tid; a < p; a += NT) {
    const double gaa = G[int64_t(a) * ld + a];
    double dg = sqrt(gaa);
    unsigned char f = 0;
    if (!(dg > 0.0) || !isfinite(dg)) {
      dg = 1.0;
      f = F_BLOCKED;
    }
    S.dg[a] = dg;
    const double u0 = (a < nwarm && !f) ? fmax(w[a], 0.0) * dg : 0.0;
    S.u[a] = u0 > 0.0 ? u0 : 0.0;
    S.flag[a] = f;
    bl = fmax(bl, f ? 0.0 : fabs(b[a] / dg));
  }
  __syncthreads();
  for (int k = tid; k < S.bk->np; k += NT) S.flag[S.plist[k]] |= F_PASSIVE;
  if (gA) {
    for (int a = tid; a < p; a += NT) S.g[a] = (S.flag[a] & F_BLOCKED) ? 0.0 : gA[a] / S.dg[a];
  } else {
    for (int a = tid; a < p; a += NT) {
      double acc = 0.0;
      for (int c = 0; c < p; ++c) acc = fma(G[int64_t(c) * ld + a], S.u[c] / S.dg[c], acc);
      S.g[a] = (S.flag[a] & F_BLOCKED) ? 0.0 : b[a] / S.dg[a] - acc / S.dg[a];
    }
  }
  __syncthreads();
  snapshot(S, p);
  double bmax;
  (void)block_argmax(bl, 0, red, &bmax);
  if (!(bmax > 0.0) || !isfinite(bmax)) return 0.0;
  return (prm.tol > 0.0 ? prm.tol : auto_tol) * bmax;
}

// Projected-gradient warm-up (step 1/L, L a Gershgorin bound of Gs).
__device__ __forceinline__ void pg_warmup(const St &S, const double *G, int64_t ld, int p, int iters, Red *red) {
  const int tid = threadIdx.x;
  double *tmp = S.rows + 2 * S.mp;
  double rowmax = 0.0;
  for (int a = tid; a < p; a += NT) {
    double acc = 0.0;
    for (int c = 0; c < p; ++c) acc += fabs(G[int64_t(c) * ld + a]) / S.dg[c];
    if (!(S.flag[a] & F_BLOCKED)) rowmax = fmax(rowmax, acc / S.dg[a]);
  }
  double Lmax;
  (void)block_argmax(rowmax, 0, red, &Lmax);
  const double step = Lmax > 0.0 ? 1.0 / Lmax : 0.0;
  for (int it = 0; it < iters; ++it) {
    __syncthreads();
    for (int a = tid; a < p; a += NT)
      tmp[a] = (S.flag[a] & F_BLOCKED) ? 0.0 : fmax(0.0, S.u[a] + step * S.g[a]) - S.u[a];
    __syncthreads();
    for (int a = tid; a < p; a += NT) {
      double acc = 0.0;
      for (int c = 0; c < p; ++c) acc = fma(G[int64_t(c) * ld + a], tmp[c] / S.dg[c], acc);
      S.g[a] -= acc / S.dg[a];
    }
    __syncthreads();
    for (int a = tid; a < p; a += NT) S.u[a] += tmp[a];
  }
  __syncthreads();
  snapshot(S, p);
}

// One refit per head.  polish: no new key; refine the last fit (p = t).
// kGlobal: the state lives in the workspace (budgets above kNnlsLdsT); else
// in LDS.  Each variant skips the heads of the other.
template <bool kGlobal>
__global__ __launch_bounds__(NT) void k_nnls_cycle(const HeadDesc *__restrict__ desc, const double *__restrict__ G,
                                                   const double *__restrict__ bvec, const double *__restrict__ gA,
                                                   double *__restrict__ w, int cycle, int kR, int polish,
                                                   NnlsParams prm, int maxp, double *__restrict__ nn_L,
                                                   int32_t *__restrict__ nn_P, int32_t *__restrict__ nn_np,
                                                   double *__restrict__ nn_vec, int32_t *__restrict__ tr_iters,
                                                   double *__restrict__ tr_weight,
                                                   int32_t *__restrict__ head_status,
                                                   int32_t *__restrict__ qr_flag,
                                                   const double *__restrict__ rpart, int nrb) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ Blk bk;
  __shared__ Red red;
  __shared__ int sh_status;
  const int h = blockIdx.x;
  const HeadDesc D = desc[h];
  if ((D.t > kNnlsLdsT) != kGlobal) return;
  // heads whose refits went to the orthogonal-factorisation path stay there
  const bool qr_ok = qr_flag && D.qr_off >= 0;
  const int qf = qr_ok ? qr_flag[h] : 0;
  // qr_flag bit 8: the exact refit follows every refit of this head and starts
  // from this refit's weights (which serve only as its warm start)
  const bool warm_only = (qf & 8) != 0;
  if (qf >= 2 && !warm_only) return;
  int64_t S0;
  int Kc;
  if (polish) {
    S0 = D.t;
    Kc = 0;
  } else {
    S0 = int64_t(cycle) * kR;
    if (S0 >= D.t) return;
    Kc = int(D.t - S0 < kR ? D.t - S0 : kR);
  }
  const int tid = threadIdx.x;
  const int p = int(S0) + Kc;
  const int np_in = S0 == 0 ? 0 : nn_np[h];
  double *Lg = nn_L + D.tt_off;
  int32_t *Pg = nn_P + D.t_off;
  // global variant: maxp > 0 means the launch gave LDS for two vectors of
  // maxp; the row slots follow them
  double *lds_rows = (kGlobal && maxp > 0 && D.t <= maxp) ? reinterpret_cast<double *>(smem) : nullptr;
  int *lds_slot = reinterpret_cast<int *>(smem + (maxp > 0 ? size_t(16) * size_t(maxp) : 0));
  double *vec_g = kGlobal ? nn_vec + D.t_off * kNnlsVecPerSlot : nullptr;
  const St S = kGlobal ? carve_global(vec_g, Lg, Pg, int(D.t), &bk, lds_rows, lds_slot)
                       : carve_lds(smem, maxp, &bk);
  if (tid == 0) {
    sh_status = 0;
    bk.np = np_in;
    bk.ctl[3] = NB;
  }
  if (!kGlobal) {
    // bring the persisted factor into LDS, eight loads in flight per thread
    const int ne = tri(np_in);
    for (int e0 = 0; e0 < ne; e0 += 8 * NT) {
      double v[8];
      static_for<0, 8>([&](auto U) {
        constexpr int u = decltype(U)::value;
        const int e = e0 + u * NT + tid;
        v[u] = Lg[e < ne ? e : ne - 1];  // unconditional load; the store below is guarded
      });
      static_for<0, 8>([&](auto U) {
        constexpr int u = decltype(U)::value;
        const int e = e0 + u * NT + tid;
        if (e < ne) S.L[e] = v[u];
      });
    }
    for (int k = tid; k < np_in; k += NT) S.plist[k] = Pg[k];
  }
  if constexpr (kGlobal && kSlotRows) {
    // the slots as the last refit left them (any order serves an empty factor)
    const int32_t *sg = persisted_slots(vec_g, int(D.t));
    for (int k = tid; k < int(D.t); k += NT) S.slot[k] = np_in > 0 ? sg[k] : k;
  }
  __syncthreads();
  // The fine test also serves every refit of a head whose Gram solve is the
  // exact refit's warm start (budgets up to 640: small factors, cheap steps): a
  // start at the minimiser leaves Lawson-Hanson a single verifying step (on the
  // 288-head stack at most 2 steps in any refit, against up to 38 from a start
  // the coarse test leaves).
  const bool fine = !(prm.tol > 0.0) && (warm_only || (polish && D.t <= kNnlsFineMaxT));
  const double tol = nnls_setup(S, G + D.tt_off, D.t, p, bvec + D.t_off, gA + D.t_off, w + D.t_off, int(S0), prm,
                                fine ? kNnlsTolFine : nnls_tol_coarse(p), &red);
  int iters = 0;
  if (tol > 0.0) {
    const int cap = prm.max_iters > 0 ? prm.max_iters : 3 * p + 30;
    nnls_core(S, G + D.tt_off, D.t, p, tol, cap, false, &red, &sh_status, &iters);
  }
  __syncthreads();
  // the fine test probes candidates whose gradients are at rounding level; a
  // dependent one among them is set aside by design, not a numeric event
  const int st = fine ? (sh_status & ~int(AMC_HS_NNLS_SINGULAR)) : sh_status;
  for (int a = tid; a < p; a += NT) w[D.t_off + a] = S.u[a] / S.dg[a];
  const int np = bk.np;
  if (!kGlobal) {
    for (int e = tid; e < tri(np); e += NT) Lg[e] = S.L[e];
    for (int k = tid; k < np; k += NT) Pg[k] = S.plist[k];
  }
  if constexpr (kGlobal && kSlotRows) {
    int32_t *sg = persisted_slots(vec_g, int(D.t));
    for (int k = tid; k < int(D.t); k += NT) sg[k] = S.slot[k];
  }
  // Does the Gram form resolve this head's minimiser?  Not when the mass is
  // fitted to a relative residual below kQrRelResid (the last residual's
  // partial sums: the KKT decisions then rest on gradients at rounding level),
  // nor when a candidate proved singular (a pivot below 1e-7 in unit-diagonal
  // form, cond(Phi_P D^-1) beyond 1e7) or the cap was hit: then this refit and
  // every later one of the head go to the orthogonal-factorisation path, which
  // reports its own status.
  bool gate = false;
  if (qr_ok && !warm_only && tol > 0.0) {
    gate = (st & int(AMC_HS_NNLS_CAP | AMC_HS_NNLS_SINGULAR)) != 0;
    if (!gate && S0 > 0 && rpart) {
      double rr = 0.0, mm = 0.0;
      for (int k = 0; k < nrb; ++k) {
        rr += rpart[(int64_t(h) * nrb + k) * 2];
        mm += rpart[(int64_t(h) * nrb + k) * 2 + 1];
      }
      gate = rr < kQrRelResid * kQrRelResid * mm;
    }
  }
  if (tid == 0) {
    nn_np[h] = np;
    if (tr_iters && !polish) tr_iters[D.cyc_off + cycle] = iters;
    if (gate) qr_flag[h] = 1;
    else if (st && head_status && !warm_only) atomicOr(head_status + h, st);
  }
  if (tr_weight)
    for (int a = tid; a < p; a += NT) tr_weight[D.t_off + a] = S.u[a] / S.dg[a];
}

#if AMC_NNLS_NT == 256  // the stand-alone solver is built once, with 256 threads
struct NnlsChunk {
  int count;
  int64_t cu_t[65];
  int64_t cu_t2[65];
};

__global__ __launch_bounds__(NT) void k_nnls_batched(NnlsChunk ch, int base, const double *__restrict__ G,
                                                     const double *__restrict__ g, double *__restrict__ w, int warm,
                                                     NnlsParams prm, int maxp, int32_t *__restrict__ iters,
                                                     int32_t *__restrict__ status) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ Blk bk;
  __shared__ Red red;
  __shared__ int sh_status;
  const int i = blockIdx.x;
  if (i >= ch.count) return;
  const int64_t t0 = ch.cu_t[i];
  const int p = int(ch.cu_t[i + 1] - t0);
  const double *Gi = G + ch.cu_t2[i];
  const St S = carve_lds(smem, maxp, &bk);
  if (threadIdx.x == 0) {
    sh_status = 0;
    bk.np = 0;
    bk.ctl[3] = NB;
  }
  __syncthreads();
  const double tol = nnls_setup(S, Gi, p, p, g + t0, nullptr, w + t0, warm ? p : 0, prm, kNnlsTolFine, &red);
  int it = 0;
  if (tol > 0.0) {
    if (prm.pg_iters > 0) pg_warmup(S, Gi, p, p, prm.pg_iters, &red);
    const int cap = prm.max_iters > 0 ? prm.max_iters : 3 * p + 30;
    nnls_core(S, Gi, p, p, tol, cap, true, &red, &sh_status, &it);
  }
  __syncthreads();
  for (int a = threadIdx.x; a < p; a += NT) w[t0 + a] = S.u[a] / S.dg[a];
  if (threadIdx.x == 0) {
    if (iters) iters[base + i] = it;
    if (status) status[base + i] = sh_status;
  }
}
#endif
