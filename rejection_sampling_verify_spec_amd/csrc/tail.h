// tail.h -- the tail of a verify call after the streaming pass (device code
// shared by the chain tail kernel and the token-tree kernels):
// the acceptance scan of a chain request and the draw of a request's final
// token.
//
// Acceptance [Primer 考点2 / 第二章]: drafted token x_i is accepted when
// u_accept[i] * p_d,i(x_i) < p_t,i(x_i), i.e. with probability
// min(1, p_t/p_d); the first rejected position n ends the scan. Greedy
// requests (T == 0) accept while x_i equals the target argmax (lowest index on
// ties) and emit the argmax at n. p(x) = 2^{(l_x - m) c} / Z, with the row
// statistics merged here in fp64 from the chunk partials of the streaming pass.
//
// Draw [Primer 考点2 residual P' = max(0, p_t - p_d) / sum; 考点4 bonus token
// from p_t when every draft passes]: inverse CDF y = min{ j : C_j > u S } in
// ascending token order. Masses are double precision in units of each row's
// maximum: e_t(j) = 2^{(l_t,j - m_t) c}, e_d(j) = 2^{(l_d,j - m_d) c},
// c = log2(e)/T, and the residual in these units is
// q_j = max(0, e_t(j) - rho e_d(j)) with rho = Z_t / Z_d, so that the chosen
// token agrees with a double-precision sequential evaluation unless u S lies
// within ~1e-13 S of a CDF boundary.
//   tile pass (one wave per tile of 2048 bf16 / 1024 fp32 tokens): tokens
//   below 2^-100 of the row maximum in both rows are left out; when few
//   remain they go straight to double precision, else through an fp32
//   triage; tokens whose masses are negligible (below 2^-50 of the row
//   maximum) and, for a residual, whose likelihood ratios are clear of the band
//   around the estimate rho~ (from the fp32 row statistics) are summed in fp32;
//   the others take double precision: fp64 masses, Z_t and Z_d, the sums over
//   tokens with e_t > rho~(1+band) e_d of (e_t - rho~ e_d) and of e_d; tokens
//   inside the band (the only ones whose residual sign the estimate cannot
//   decide) are summed in groups of equal logit difference l_t - l_d, which
//   share one likelihood ratio.
//   pick: exact rho = Z_t / Z_d, exact tile masses dpos + (rho~ - rho) bpos +
//   sum over groups of max(0, sum e_t - rho sum e_d) (tiles whose groups did
//   not fit, or every tile when rho leaves the band, are recomputed token by
//   token), a scan over tiles for the one holding u S, and a fixed-order fp64
//   scan of that tile.
//
// A chain request's tail runs in a few workgroups of NW waves: each runs the
// acceptance scan, the waves of all of them take the tiles in turn, and the
// last workgroup to finish runs the pick. Token trees run the same tile pass
// and pick as kernels of their own after the tree acceptance kernel.
#pragma once

#include "specverify.h"
#include "sv_internal.h"

namespace sv {

// Wave64 reductions and scans on DPP lane moves (gfx9 controls: row_shr:n =
// 0x110 + n inside rows of 16 lanes, row_bcast:15 = 0x142 into rows 1 and 3,
// row_bcast:31 = 0x143 into rows 2 and 3). Every lane of the wave must be
// active. The association order is fixed, so results are reproducible; the
// totals are read from lane 63 and are the same in every lane.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, ROW_MASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, ROW_MASK, 0xf, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Inclusive prefix sum over the 64 lanes (lanes without a source add +0).
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_f64<0x111, 0xf>(v);
  v += dpp_f64<0x112, 0xf>(v);
  v += dpp_f64<0x114, 0xf>(v);
  v += dpp_f64<0x118, 0xf>(v);
  v += dpp_f64<0x142, 0xa>(v);
  v += dpp_f64<0x143, 0xc>(v);
  return v;
}

__device__ __forceinline__ double lane_f64(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, lane), hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Sum over the wave, the same value in every lane.
__device__ __forceinline__ double wave_sum(double v) { return lane_f64(wave_incl_scan(v), 63); }

// min / max of an int over the wave.
template <bool MAX>
__device__ __forceinline__ int wave_minmax(int v) {
  constexpr int id = MAX ? (int)0x80000000 : 0x7fffffff;
  auto op = [](int a, int b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x111, 0xf, 0xf, false));
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x112, 0xf, 0xf, false));
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x114, 0xf, 0xf, false));
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x118, 0xf, 0xf, false));
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x142, 0xa, 0xf, false));
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(v, 63);
}

constexpr int kList = 64;             // undecided tokens collected per tile
constexpr int kSparse = 4;            // live tokens per lane up to which a tile triages them one by one
constexpr int kMaxPos = SV_MAX_GAMMA + 1;
constexpr int kRowLanes = 8;          // lanes merging one row's chunk partials (DPP groups of 8)

template <int DT, int NW> struct TileGeom {
  static constexpr int nt = NW * 64;                       // threads of the workgroup
  static constexpr int tok = TileTok<DT>::value;          // tokens per tile
  static constexpr int epl = tok / 64;                     // tokens per lane (wave-owned tile)
  static constexpr int nv = epl / Elem<DT>::kPerVec;       // 16-byte vectors per lane
  static constexpr int bt = tok / nt;                      // tokens per thread (workgroup-owned tile)
  static_assert(nv == 4, "four 16-byte vectors per lane");
  static_assert(bt * nt == tok, "a workgroup tile splits evenly over the threads");
};

// ---------------------------------------------------------------------------
// Shared memory of a tail workgroup.

template <int NW>
struct TileLists {  // per-wave lists of undecided tokens of the exact pass
  double dl[NW][kList], et[NW][kList], ed[NW][kList];
};

// Tile records of one request copied into LDS by the pick (rows with more
// tiles read them from global memory).
constexpr int kPickStage = 256;
constexpr int kRecWords = (int)(sizeof(TileRec) / 8);

template <int NW>
struct PickSpace {
  double red[NW];
  double Zt, Zd, W, thr;
  int tile, last_mode, any_exact, res;
  int smin[NW], smax[NW];
  uint64_t rw[kPickStage * kRecWords];  // staged records, word w of tile k at k * kRecWords + w
};

// Partials of one chain request kept in LDS by the acceptance scan (requests
// with more rows times chunks read them from global memory).
constexpr int kPartCache = 1024;

struct AcceptSpace {
  // per position i <= g
  int x[kMaxPos];
  float ua[kMaxPos], us[kMaxPos], lt[kMaxPos], ld[kMaxPos], pt[kMaxPos], pd[kMaxPos];
  // per row: target rows 0..g, then draft rows 0..g-1
  double gap[kMaxPos];  // p_d(x_i) - p_t(x_i)
  double rz[2 * kMaxPos];
  float rm[2 * kMaxPos];
  int ridx[2 * kMaxPos];
  unsigned char rok[2 * kMaxPos];
  // the request's partials: row r (target rows 0..g, then draft rows) at r * nchunk
  Partial pc[kPartCache];
};

// LDS copy of the waves' tiles (raw 16-byte vectors [u][lane]) for the per-token
// double-precision fixup; residual draws also stage the draft row.
template <int NW>
struct TileStage {
  uint4 t[NW][4][64];
  uint4 d[NW][4][64];
};

template <int NW>
struct TileSpace {
  TileLists<NW> lists;
  TileStage<NW> stage;
};

// ---------------------------------------------------------------------------
// The sampling job in scalar registers.

// The job from shared memory into scalar registers (it is the same for every
// thread; a plain load would hold it in vector registers).
__device__ __forceinline__ SampleJob uniform_job(const SampleJob& src) {
  static_assert(sizeof(SampleJob) % 4 == 0, "job of 32-bit words");
  constexpr int nw = sizeof(SampleJob) / 4;
  int w[nw];
  const int* p = reinterpret_cast<const int*>(&src);
#pragma unroll
  for (int i = 0; i < nw; ++i) w[i] = __builtin_amdgcn_readfirstlane(p[i]);
  SampleJob J;
  __builtin_memcpy(&J, w, sizeof(J));
  return J;
}

// ---------------------------------------------------------------------------
// Tile records pass between the workgroups of a request (which may sit on
// different XCDs, each with its own L2): their 64-bit words are written and
// read as device-scope atomic accesses, coherent without cache write-backs.

constexpr int kRecZt = 0, kRecZd = 1, kRecDpos = 2, kRecBpos = 3, kRecNgrp = 4, kRecGet = 5, kRecGed = 5 + kGrp;

__device__ __forceinline__ void rec_store(TileRec* R, int word, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(R) + word, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t rec_load(const TileRec* R, int word) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<TileRec*>(R)) + word, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t f64_word(double v) { return (uint64_t)__double_as_longlong(v); }
__device__ __forceinline__ uint64_t ngrp_word(int ng) { return (uint64_t)(uint32_t)ng; }

// A record whose fields are wave-uniform, except the group sums: lane g < ng
// holds group g's (gt, gd). Lanes 0 .. kRecWords-1 store one word each.
__device__ __forceinline__ void write_rec(TileRec* rec, double zt, double zd, double dp, double bp, int ng, double gt,
                                          double gd, int lane) {
  const int g = lane < kRecGed ? lane - kRecGet : lane - kRecGed;
  const double gtl = __shfl(gt, g & 63, 64), gdl = __shfl(gd, g & 63, 64);
  uint64_t word = 0;
  if (lane == kRecZt) word = f64_word(zt);
  else if (lane == kRecZd) word = f64_word(zd);
  else if (lane == kRecDpos) word = f64_word(dp);
  else if (lane == kRecBpos) word = f64_word(bp);
  else if (lane == kRecNgrp) word = ngrp_word(ng);
  else if (lane >= kRecGet && lane < kRecGed) word = f64_word(ng > g ? gtl : 0.0);
  else if (lane >= kRecGed && lane < kRecGed + kGrp) word = f64_word(ng > g ? gdl : 0.0);
  if (lane < kRecWords) rec_store(rec, lane, word);
}

// The record of a tile inside a chunk whose tiles are not read (lane 0): the
// chunk's first tile carries the whole chunk's masses (target, and draft for a
// residual draw), the others none; the residual mass of the tile is 0.
__device__ __forceinline__ void write_skipped_rec(TileRec* rec, bool head, double chunk_mass_t,
                                                  double chunk_mass_d) {
  rec_store(rec, kRecZt, f64_word(head ? chunk_mass_t : 0.0));
  rec_store(rec, kRecZd, f64_word(head ? chunk_mass_d : 0.0));
  rec_store(rec, kRecDpos, f64_word(0.0));
  rec_store(rec, kRecBpos, f64_word(0.0));
  rec_store(rec, kRecNgrp, ngrp_word(head ? kRecChunkHead : kRecChunkBody));
}

// ---------------------------------------------------------------------------
// Token masses of the draw.

// 2^a in double precision for -1100 <= a <= 0 (the caller keeps a in range;
// NaN propagates through the arithmetic), with tab[j] = 2^{j/64}:
// a = n + j/64 + r with n an integer, 0 <= j < 64 and |r| <= 1/128 (r is exact:
// a and k/64 are within a factor of two of each other or r is the tiny rest),
// and 2^r = exp(r ln 2) by its Taylor series to degree 5 (truncation below
// 4e-17 relative). About 3 ulp in all.
// p * r + c as the three-operand v_fma_f64 with the constant coefficient c in
// a scalar register pair (one scalar operand per instruction): the compiler
// otherwise picks the accumulating form, which overwrites its addend and so
// copies the coefficient into fresh vector registers before every step, or
// keeps every coefficient in vector registers across the tile loops.
__device__ __forceinline__ double fma3_f64(double p, double r, double c) {
  double d;
  __asm__("v_fma_f64 %0, %1, %2, %3" : "=v"(d) : "v"(p), "v"(r), "s"(c));
  return d;
}
// The first step, c1 * r + c0, with c1 in a scalar and c0 in a vector register
// pair (both constants; a scalar pair for each would exceed the one scalar
// operand an instruction may read).
__device__ __forceinline__ double fma_first_f64(double r, double c1, double c0) {
  double d;
  __asm__("v_fma_f64 %0, %1, %2, %3" : "=v"(d) : "v"(r), "s"(c1), "v"(c0));
  return d;
}

// The two constants exp2_tab reads from vector registers (the shifter and the
// degree-4 coefficient). Built by pinned_exp2() before a loop, they are opaque
// to the compiler, which otherwise rebuilds them for every token.
struct Exp2Regs {
  double shift, c4;
};
__device__ __forceinline__ Exp2Regs pinned_exp2() {
  Exp2Regs K{0x1.8p52, 0x1.3b2ab6fba4e77p-7};
  __asm__ volatile("" : "+v"(K.shift), "+v"(K.c4));
  return K;
}

__device__ __forceinline__ double exp2_tab(double a, const double* tab, const Exp2Regs& K) {
  // k = rint(64 a) by the shifter 1.5 * 2^52 (|64 a| < 2^51): the low 32 bits
  // of t hold k as a two's-complement int
  double t;
  __asm__("v_fma_f64 %0, %1, %2, %3" : "=v"(t) : "v"(a), "s"(64.0), "v"(K.shift));
  const int ki = (int)(uint32_t)(uint64_t)__double_as_longlong(t);
  const double tv = tab[ki & 63];  // (read before the polynomial, which then covers its latency)
  const double k = t - 0x1.8p52;
  const double r = __builtin_fma(k, -0.015625, a);
  double p = fma_first_f64(r, 0x1.5d87fe78a6731p-10, K.c4);  // ln2^5 / 5!, ln2^4 / 4!
  p = fma3_f64(p, r, 0x1.c6b08d704a0c0p-5);  // ln2^3 / 3!
  p = fma3_f64(p, r, 0x1.ebfbdff82c58fp-3);  // ln2^2 / 2!
  p = fma3_f64(p, r, 0x1.62e42fefa39efp-1);  // ln2
  p = __builtin_fma(p, r, 1.0);
  return __builtin_ldexp(tv * p, ki >> 6);
}
__device__ __forceinline__ double exp2_tab(double a, const double* tab) {
  return exp2_tab(a, tab, Exp2Regs{0x1.8p52, 0x1.3b2ab6fba4e77p-7});
}

// Mass 2^{(l - m) c} of one token in double precision (c64 = c), in units of
// its row's maximum. Arguments below -1100 (masses that are 0 in fp64, and
// l = -inf) are raised to -1100, inside exp2_tab's range, by one max rather
// than a branch. A NaN argument would also give 0, but no draw reads a row
// with a NaN or +inf logit: the streaming pass flags such rows and their
// requests fail before any draw.
__device__ __forceinline__ double emass_t(float l, float m, double c64, const double* tab, const Exp2Regs& K) {
  return exp2_tab(fmax(((double)l - (double)m) * c64, -1100.0), tab, K);
}
__device__ __forceinline__ double emass_t(float l, float m, double c64, const double* tab) {
  return exp2_tab(fmax(((double)l - (double)m) * c64, -1100.0), tab);
}

// ---------------------------------------------------------------------------
// Acceptance scan of chain request b by a whole workgroup.

// Merge the chunk partials of one row by the kRowLanes lanes of a group (lane
// `sub` takes chunks sub, sub + kRowLanes, ...; src(k) gives chunk k). The
// maximum keeps the lowest token index among equal values (chunks are in
// ascending token order); Z is the fixed-order sum of s_k 2^{(m_k - M) c}.
// Every lane of the group ends with the same values.
template <typename Src>
__device__ __forceinline__ void merge_row_group(Src src, int nchunk, double c, bool greedy, int sub, float& M,
                                                int& idx, double& Z, bool& ok) {
  M = -INFINITY;
  idx = -1;
  bool bad = false;
  for (int k = sub; k < nchunk; k += kRowLanes) {
    const Partial q = src(k);
    bad |= partial_bad(q, greedy);
    if (q.m > M) { M = q.m; idx = partial_idx(q); }
  }
  // exchanges inside the group of 8 lanes: xor 1 and xor 2 (quad permutes),
  // then the mirrored lane of the other quad
  auto step = [&](auto mv) {
    const float M2 = __int_as_float(mv(__float_as_int(M)));
    const int i2 = mv(idx);
    bad |= mv((int)bad) != 0;
    if (M2 > M || (M2 == M && (unsigned)i2 < (unsigned)idx)) { M = M2; idx = i2; }
  };
  step([](int v) { return __builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, false); });
  step([](int v) { return __builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, false); });
  step([](int v) { return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false); });
  ok = !bad && M > -INFINITY && M < INFINITY;
  Z = 0.0;
  if (greedy || !ok) return;
  for (int k = sub; k < nchunk; k += kRowLanes) {
    const Partial q = src(k);
    if (q.m > -INFINITY) Z += (double)partial_s(q) * exp2_f64(((double)q.m - (double)M) * c);
  }
  Z += dpp_f64<0xb1, 0xf>(Z);
  Z += dpp_f64<0x4e, 0xf>(Z);
  Z += dpp_f64<0x141, 0xf>(Z);
  ok = Z > 0.0 && Z < 1e308;
}

struct ChainArgs {
  Layout L;
  const int32_t* tokens;
  const float* ua;
  const float* us;
  const float* temperature;
  const Partial* part;
  int nchunk;
  int chunk_vecs;  // 16-byte vectors per chunk of the streaming pass
  int32_t* num_acc;
  float* diag;
};

// Rows of chain request b: g drafted positions, target rows t0 .. t0+g, draft
// rows d0 .. d0+g-1 (ragged: through cu_gamma, whose validity the caller has
// established).
struct ChainRows {
  int g;
  long long t0, d0;
};
__device__ __forceinline__ ChainRows chain_rows(const Layout& L, int b) {
  if (L.mode == LAYOUT_RAGGED) {
    const long long d0 = L.cu[b];
    return ChainRows{(int)(L.cu[b + 1] - d0), d0 + b, d0};
  }
  return ChainRows{L.gamma, (long long)b * (L.gamma + 1), (long long)b * L.gamma};
}

// Row chunks whose tiles are not read again (rows 16-byte aligned, so that the
// streaming pass's chunks start on tile boundaries). A chunk whose maximum
// lies more than -kTinyExp below its row maximum (in units of the exponent
// argument) holds only negligible masses, every one below 2^-50 of the row
// maximum, and at most 2^-36 in all:
//   bonus draw: the chunk's mass comes from its partial, s 2^{(m_chunk -
//     m_row) c}, accurate to the fp32 sum of the streaming pass (relative 1e-6
//     of a total below 2^-36);
//   residual draw: chunks negligible in both rows; their Z_t and Z_d parts
//     come from the partials in the same way, and their residual mass, which
//     lies between 0 and the chunk's target mass, is taken as 0 -- only while
//     the sum of those target masses stays below 1e-12 of a lower bound of the
//     residual total, so that no CDF position moves by more than 1e-12 S. The
//     bound is the larger of Z_t (p_d(x_n) - p_t(x_n)) and half the summed
//     chunk differences |Z_t P_t(chunk) - rho Z_d P_d(chunk)| (the residual
//     total is half the total-variation sum, which merging tokens into chunks
//     can only decrease), less a margin for the fp32 partial sums.
// Wave 0 only: sets J.skip (bit k = chunk k) and J.chunk_tiles, and
// mass_t[k] (and mass_d[k]) for the skipped chunks.
// cache_t / cache_d: LDS copies of the partials of the drawn rows, or null.
template <int DT>
__device__ __forceinline__ void find_skipped_chunks(const void* tgt, const void* dft, int V, const Partial* part,
                                                    long long RT, int nchunk, int chunk_vecs, SampleJob& J,
                                                    const Partial* cache_t, const Partial* cache_d,
                                                    double* mass_t, double* mass_d, int lane) {
  constexpr int es = sizeof(typename Elem<DT>::T);
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int tok = TileTok<DT>::value;
  const long long ctok = (long long)chunk_vecs * epv;
  const bool res = J.kind == JOB_RESIDUAL;
  auto aligned = [&](const void* base, long long row) {
    return (reinterpret_cast<uintptr_t>(reinterpret_cast<const char*>(base) + (size_t)row * (size_t)V * es) & 15u) ==
           0;
  };
  if (!(J.kind != JOB_NONE && aligned(tgt, J.trow) && (!res || aligned(dft, J.drow)) && nchunk <= 64 &&
        nchunk > 1 && ctok % tok == 0))
    return;
  // chunk masses relative to a row maximum, from the partial; tiny = negligible
  auto chunk = [&](long long prow, const Partial* cache, float m_row, bool& tiny) -> double {
    const Partial q = cache ? cache[lane] : read_partial(part + prow * nchunk + lane);
    tiny = q.m == -INFINITY || (q.m - m_row) * J.c32 < kTinyExp;
    if (q.m == -INFINITY) return 0.0;
    return (double)partial_s(q) * exp2_f64(((double)q.m - (double)m_row) * (double)J.c32);
  };
  bool tiny = false;
  double mt = 0.0, md = 0.0;
  if (lane < nchunk) {
    mt = chunk(J.trow, cache_t, J.mt, tiny);
    if (res) {
      bool tiny_d = false;
      md = chunk(RT + J.drow, cache_d, J.md, tiny_d);
      tiny = tiny && tiny_d;
    }
    mass_t[lane] = mt;
    if (res) mass_d[lane] = md;
  }
  if (res) {
    const double dropped = wave_sum(tiny ? mt : 0.0);
    const double dtv = mt - J.rho * md, tv_margin = 2e-6 * (mt + J.rho * md);
    const double tv = wave_sum(lane < nchunk ? fmax(0.0, fabs(dtv) - tv_margin) : 0.0);
    const double slow = fmax(J.slow, 0.5 * tv);
    if (!(dropped <= 1e-12 * slow)) return;
  }
  const unsigned long long mask = __ballot(tiny);
  if (lane == 0) {
    J.skip = mask;
    J.chunk_tiles = (int)(ctok / tok);
  }
}

// Writes the request's accepted tokens (and the greedy token), num_accepted and
// the diagnostics, and leaves the sampling job in `job`. `usable` false marks
// the request as failed without reading anything (malformed layout).
//
// Latency matters here more than work: the loads that do not depend on each
// other (the thread's first drafted token, the request's chunk partials, the
// temperature, the uniforms) are issued together, then the two logits at the
// token; the partials are merged from an LDS copy, which also serves the
// chunk masses of the draw.
template <int DT, int NW>
__device__ __forceinline__ void accept_chain(const void* __restrict__ tgt, const void* __restrict__ dft, int V, const ChainArgs& A,
                             int b, const ChainRows& R, bool usable, bool write, int32_t* __restrict__ orow,
                             int out_width, AcceptSpace& P, SampleJob& job, double* mass_t, double* mass_d, int& s_n,
                             int& s_bad) {
  constexpr int NT = NW * 64;
  constexpr int kPer = (kPartCache + NT - 1) / NT;
  const int tid = threadIdx.x;
  const Layout& L = A.L;
  const int g = usable ? R.g : 0;
  const long long t0 = R.t0, d0 = R.d0;
  const int nchunk = A.nchunk;
  const int nrows = 2 * g + 1;  // target rows 0..g, then draft rows 0..g-1
  const bool cached = usable && (long long)nrows * nchunk <= kPartCache;
  auto prow_of = [&](int r) -> long long { return r <= g ? t0 + r : L.RT + d0 + (r - g - 1); };
  if (tid == 0) {
    s_n = 0x7fffffff;
    s_bad = 0;
  }

  // --- independent loads, in flight together
  const int i0 = tid;  // the thread's first position
  int x0 = 0;
  if (usable && i0 < g) x0 = A.tokens[d0 + i0];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = tid + k * NT;
    if (cached && e < nrows * nchunk) {
      const int r = e / nchunk;
      P.pc[e] = read_partial(A.part + prow_of(r) * nchunk + (e - r * nchunk));
    }
  }
  const float T = A.temperature[b];
  float us0 = 0.f, ua0 = 0.f, lt0 = 0.f, ld0 = 0.f;
  if (usable && i0 <= g) us0 = A.us[t0 + i0];
  if (usable && i0 < g) ua0 = A.ua[d0 + i0];
  // the logits at the drafted token need only the token
  if (usable && i0 < g && x0 >= 0 && x0 < V) {
    lt0 = Elem<DT>::at(tgt, (t0 + i0) * (long long)V + x0);
    ld0 = Elem<DT>::at(dft, (d0 + i0) * (long long)V + x0);
  }
  const bool bad0 = !usable || !temperature_ok(T);
  const bool greedy = T == 0.0f;
  const float c32 = bad0 || greedy ? 0.0f : c32_of(T);
  const double c = (double)c32;

  // --- per-position inputs into LDS (positions past the first NT: gamma = NT)
  bool lbad = false;
  if (!bad0) {
    auto put = [&](int i, int x, float u_s, float u_a, float lt, float ld) {
      const bool xok = i == g || (x >= 0 && x < V);
      if (!greedy) lbad |= !uniform_ok(u_s) || (i < g && !uniform_ok(u_a));
      lbad |= !xok;
      P.x[i] = x;
      P.ua[i] = greedy ? 0.f : u_a;
      P.us[i] = greedy ? 0.f : u_s;
      P.lt[i] = greedy ? 0.f : lt;
      P.ld[i] = greedy ? 0.f : ld;
    };
    if (i0 <= g) put(i0, x0, us0, ua0, lt0, ld0);
    for (int i = i0 + NT; i <= g; i += NT) {
      int x = 0;
      float u_a = 0.f, lt = 0.f, ld = 0.f;
      if (i < g) {
        x = A.tokens[d0 + i];
        u_a = A.ua[d0 + i];
        if (x >= 0 && x < V) {
          lt = Elem<DT>::at(tgt, (t0 + i) * (long long)V + x);
          ld = Elem<DT>::at(dft, (d0 + i) * (long long)V + x);
        }
      }
      put(i, x, A.us[t0 + i], u_a, lt, ld);
    }
  }
  __syncthreads();

  // --- row statistics: target rows 0..g, then (T > 0) draft rows 0..g-1
  if (!bad0) {
    if (lbad) s_bad = 1;
    const int nr = (g + 1) + (greedy ? 0 : g);
    const int grp = tid / kRowLanes, sub = tid % kRowLanes;
    for (int r = grp; r < nr; r += NT / kRowLanes) {
      float M;
      int idx;
      double Z;
      bool ok;
      if (cached) {
        const Partial* pc = P.pc + r * nchunk;
        merge_row_group([&](int k) { return pc[k]; }, nchunk, c, greedy, sub, M, idx, Z, ok);
      } else {
        const Partial* pg = A.part + prow_of(r) * nchunk;
        merge_row_group([&](int k) { return read_partial(pg + k); }, nchunk, c, greedy, sub, M, idx, Z, ok);
      }
      if (sub == 0) {
        P.rm[r] = M;
        P.rz[r] = Z;
        P.ridx[r] = idx;
        P.rok[r] = ok;
      }
    }
  }
  __syncthreads();

  // --- decisions per position; validation covers every position
  if (!bad0) {
    bool pbad = false;
    int rej = 0x7fffffff;
    for (int i = tid; i <= g; i += NT) {
      bool pb = !P.rok[i];
      if (i < g && !greedy) pb |= !P.rok[g + 1 + i];
      pbad |= pb;
      if (i < g && !pb) {
        const int x = P.x[i];
        bool reject;
        if (greedy) {
          reject = x != P.ridx[i];
        } else {
          const double pt = exp2_f64(((double)P.lt[i] - (double)P.rm[i]) * c) / P.rz[i];
          const double pd = exp2_f64(((double)P.ld[i] - (double)P.rm[g + 1 + i]) * c) / P.rz[g + 1 + i];
          reject = !((double)P.ua[i] * pd < pt);
          P.pt[i] = (float)pt;
          P.pd[i] = (float)pd;
          P.gap[i] = pd - pt;
        }
        if (reject && i < rej) rej = i;
      }
    }
    if (pbad) s_bad = 1;
    if (rej != 0x7fffffff) atomicMin(&s_n, rej);
  }
  __syncthreads();

  // --- outputs and the sampling job
  const bool bad = bad0 || s_bad != 0;
  const int n = bad ? 0 : min(s_n, g);
  const bool draw = !bad && !greedy;  // column n then receives the drawn token
  for (int k = tid; write && k < out_width; k += NT) {
    int v = -1;
    if (!bad) {
      if (k < n) v = P.x[k];
      else if (k == n && greedy) v = P.ridx[n];
    }
    if (!(draw && k == n)) orow[k] = v;
  }
  if (write && tid == 0) A.num_acc[b] = bad ? -1 : n;
  if (write && A.diag && usable)
    for (int i = tid; i < R.g; i += NT) {
      const float qnan = __uint_as_float(0x7fc00000u);
      A.diag[2 * (d0 + i)] = bad || greedy ? qnan : P.pt[i];
      A.diag[2 * (d0 + i) + 1] = bad || greedy ? qnan : P.pd[i];
    }
  if (tid < 64) {  // wave 0: the sampling job and the chunks its draw skips
    SampleJob J;
    J.kind = (bad || greedy) ? JOB_NONE : (n < g ? JOB_RESIDUAL : JOB_BONUS);
    J.pos = n;
    J.trow = t0 + n;
    J.drow = d0 + n;
    J.c64 = bad || greedy ? 0.0 : c64_of(T);
    J.c32 = c32;
    J.skip = 0ull;
    J.chunk_tiles = 0;
    J.pad = 0;
    J.u = bad || greedy ? 0.0f : P.us[n];
    J.mt = bad ? 0.0f : P.rm[n];
    J.md = J.kind == JOB_RESIDUAL ? P.rm[g + 1 + n] : 0.0f;
    J.rho = J.kind == JOB_RESIDUAL ? P.rz[n] / P.rz[g + 1 + n] : 0.0;
    // the residual total is at least p_d(x_n) - p_t(x_n) > 0 in probability
    // units (its positive and negative parts are equal, and x_n is in the
    // negative part), i.e. Z_t (p_d - p_t) in units of the target row maximum;
    // a relative 1e-6 margin covers the rounding of the two probabilities
    J.slow = J.kind == JOB_RESIDUAL ? P.rz[n] * (P.gap[n] - 1e-6 * (double)P.pd[n]) : 0.0;
    find_skipped_chunks<DT>(tgt, dft, V, A.part, L.RT, nchunk, A.chunk_vecs, J, cached ? P.pc + n * nchunk : nullptr,
                            cached ? P.pc + (g + 1 + n) * nchunk : nullptr, mass_t, mass_d, tid);
    if (tid == 0) job = J;
  }
  __syncthreads();
}

// Tile k lies in a chunk whose tiles are not read.
__device__ __forceinline__ bool tile_skipped(const SampleJob& J, int k) {
  return J.skip && ((J.skip >> (k / J.chunk_tiles)) & 1ull);
}

// ---------------------------------------------------------------------------
// Tile loads.

// Raw bits of one logit and of -inf, per storage type.
template <int DT> __device__ __forceinline__ uint32_t raw_at(const void* rowp, int j);
template <> __device__ __forceinline__ uint32_t raw_at<0>(const void* rowp, int j) {
  return reinterpret_cast<const uint32_t*>(rowp)[j];
}
template <> __device__ __forceinline__ uint32_t raw_at<1>(const void* rowp, int j) {
  return reinterpret_cast<const uint16_t*>(rowp)[j];
}
template <int DT> struct NegInf;
template <> struct NegInf<0> { static constexpr uint32_t bits = 0xff800000u; };
template <> struct NegInf<1> { static constexpr uint32_t bits = 0xff80u; };

// One 16-byte vector of tokens j .. j+epv-1 (element order of unpack<DT>);
// tokens at or beyond V read as -inf. A vector load when the vector is in range
// and 16-byte aligned, token by token otherwise.
template <int DT>
__device__ __forceinline__ uint4 load_vec(const void* rowp, int j, int V) {
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const char* p = reinterpret_cast<const char*>(rowp) + (size_t)j * es;
  if (j + epv <= V && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) return *reinterpret_cast<const uint4*>(p);
  uint32_t bits[epv];
#pragma unroll
  for (int e = 0; e < epv; ++e) bits[e] = j + e < V ? raw_at<DT>(rowp, j + e) : NegInf<DT>::bits;
  if constexpr (DT == 1)
    return make_uint4(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16), bits[4] | (bits[5] << 16),
                      bits[6] | (bits[7] << 16));
  else
    return make_uint4(bits[0], bits[1], bits[2], bits[3]);
}

// A wave's tile: lane l holds vectors u*64 + l (u < nv) of the tile, i.e. tokens
// j0 + (u*64 + l)*epv + e.
template <int DT>
__device__ __forceinline__ void load_tile_wave(const void* rowp, int j0, int V, int lane, uint4 (&w)[4]) {
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int es = sizeof(typename Elem<DT>::T);
  constexpr int tok = TileTok<DT>::value;
  const char* p = reinterpret_cast<const char*>(rowp) + (size_t)j0 * es;
  if (j0 + tok <= V && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = reinterpret_cast<const uint4*>(p)[u * 64 + lane];
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = load_vec<DT>(rowp, j0 + (u * 64 + lane) * epv, V);
  }
}

// ---------------------------------------------------------------------------
// Tile pass.

// A lane's double-precision sums over its flagged tokens.
struct ExactAcc {
  double zt, zd, dp, bp;
  int n;  // undecided tokens seen (wave-uniform)
};

// The sums of one token in double precision; returns whether it is undecided
// (inside the band around rho~), with its masses in et and ed.
template <bool RES>
__device__ __forceinline__ bool exact_sums(float xt, float xd, const SampleJob& J, double hi, double lo, ExactAcc& A,
                                           const double* tab, const Exp2Regs& K, double& et, double& ed) {
  et = emass_t(xt, J.mt, J.c64, tab, K);
  A.zt += et;
  if (!RES) return false;
  ed = emass_t(xd, J.md, J.c64, tab, K);
  A.zd += ed;
  // a token on the positive side adds et - rho ed and ed, as fma(1, ., .);
  // the others add nothing, as fma(0, ., .) (masses are finite): the same
  // sums as adding under a branch, without one
  const bool pos = et > hi * ed;
  const double pf = pos ? 1.0 : 0.0;
  A.dp = __builtin_fma(pf, __builtin_fma(-J.rho, ed, et), A.dp);
  A.bp = __builtin_fma(pf, ed, A.bp);
  return !pos && et > 0.0 && et >= lo * ed;
}

// Appends this step's undecided tokens to the wave's list, in lane order.
template <int NW>
__device__ __forceinline__ void append_undecided(bool und, float xt, float xd, double et, double ed,
                                                 unsigned long long below, ExactAcc& A, TileLists<NW>& L, int wv) {
  const unsigned long long m = __ballot(und);
  if (m) {
    const int slot = A.n + __builtin_popcountll(m & below);
    if (und && slot < kList) {
      L.dl[wv][slot] = (double)xt - (double)xd;
      L.et[wv][slot] = et;
      L.ed[wv][slot] = ed;
    }
    A.n += __builtin_popcountll(m);
  }
}

// Double-precision treatment of one flagged token (has == false: this lane has
// none left this step, but still takes part in the wave ballot).
template <bool RES, int NW>
__device__ __forceinline__ void exact_token(bool has, float xt, float xd, const SampleJob& J, double hi, double lo,
                                            unsigned long long below, ExactAcc& A, TileLists<NW>& L, int wv,
                                            const double* tab, const Exp2Regs& K) {
  double et = 0.0, ed = 0.0;
  bool und = false;
  if (has) und = exact_sums<RES>(xt, xd, J, hi, lo, A, tab, K, et, ed);
  if (RES) append_undecided<NW>(und, xt, xd, et, ed, below, A, L, wv);
}

// Token e of a staged 16-byte vector, read from LDS.
template <int DT>
__device__ __forceinline__ float staged_at(const uint4& v, int e) {
  if constexpr (DT == 1) {
    const uint16_t bits = reinterpret_cast<const uint16_t*>(&v)[e];
    return __uint_as_float((uint32_t)bits << 16);
  } else {
    return reinterpret_cast<const float*>(&v)[e];
  }
}

// Token i (u = i / epv, e = i % epv) of a lane's four 16-byte vectors, by
// selects on the registers (a lane-dependent index).
template <int DT>
__device__ __forceinline__ float token_at(uint4 w0, uint4 w1, uint4 w2, uint4 w3, int i) {
  constexpr int epv = Elem<DT>::kPerVec;
  const int u = i / epv, e = i % epv;
  const uint4 v = u == 0 ? w0 : u == 1 ? w1 : u == 2 ? w2 : w3;
  if constexpr (DT == 1) {
    const int q = e >> 1;
    const uint32_t d = q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
    return __uint_as_float((e & 1) ? (d & 0xffff0000u) : (d << 16));
  } else {
    const uint32_t d = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
    return __uint_as_float(d);
  }
}

// Pass over one tile by one wave; writes the tile record. The lane holds the
// tile's 16-byte vectors u*64 + lane (u < 4) in wt (and wd); its token (u, e)
// is token j0 + (u*64 + lane)*epv + e.
//
// Tokens below 2^kDropExp of the row maximum in both rows are left out (masses
// below the resolution of the sums). When no lane holds more than kSparse
// of the others, each is picked from the registers and goes through fp32 on
// its own. Otherwise every token of a vector holding one goes through fp32. A token whose mass is below 2^-50 of its
// row maximum in both rows (fp32 argument a < kTinyExp) and, for a residual,
// whose likelihood ratio lies outside twice the band around rho~ contributes
// terms whose fp32 rounding is below 2^-70 of the row maximum: it is summed,
// and for a residual decided, in fp32. Every other token is flagged. The
// lane's flagged tokens are then taken one per step in double precision (fp64
// masses; the band decision in fp64; undecided tokens appended to a list in a
// fixed order (step, lane) through wave ballots), with their logits read back
// from an LDS copy of the tile. Near one-hot rows flag a handful of tokens per
// row; rows where every mass is significant flag every token.
//
// next() is called once the tile's registers wt / wd are free (after the
// triage and the per-token fixups), so that the caller can issue the loads of
// its next tile into them while this one's sums and record are finished.
template <int DT, bool RES, int NW, typename Next>
__device__ __forceinline__ void tile_pass(uint4 (&wt)[4], uint4 (&wd)[4], const SampleJob& J, TileRec* rec,
                                          TileSpace<NW>& TS, const double* tab, int wv, int lane, Next next) {
  constexpr int epv = Elem<DT>::kPerVec;
  constexpr int nv = 4;
  static_assert(nv * epv <= 32, "one flag bit per token of the lane");
  TileLists<NW>& L = TS.lists;
  TileStage<NW>& G = TS.stage;
  const float mt = J.mt, md = J.md, c32 = J.c32;
  float st = 0.f, sd = 0.f, sdp = 0.f, sbp = 0.f;
  uint32_t flags = 0u;
  // Live tokens: at or above 2^kDropExp of the row maximum in either row, as
  // logit thresholds; the others are left out (vectors without one are not
  // unpacked further).
  const float tt = mt + kDropExp / c32, td = RES ? md + kDropExp / c32 : 0.f;
  uint32_t live = 0u;
  // vectors u whose every token, in every lane, lies at or above 2^kTinyExp of
  // its row maximum in the target row (or the draft row of a residual): the
  // triage would flag each of them and add +0 to every sum, so it skips them.
  // (x - m) * c is monotone in x in fp32 as in exact arithmetic, so the test on
  // the vector's smallest logit is the triage's own test on every token.
  uint32_t dense = 0u;  // wave-uniform, bit u
#pragma unroll
  for (int u = 0; u < nv; ++u) {
    float xt[epv], xd[epv];
    unpack<DT>(wt[u], xt);
    if (RES) unpack<DT>(wd[u], xd);
    float vt = xt[0], vd = RES ? xd[0] : 0.f, nt = xt[0], nd = RES ? xd[0] : 0.f;
#pragma unroll
    for (int e = 1; e < epv; ++e) {
      vt = fmaxf(vt, xt[e]);
      nt = fminf(nt, xt[e]);
      if (RES) {
        vd = fmaxf(vd, xd[e]);
        nd = fminf(nd, xd[e]);
      }
    }
    if (__all((nt - mt) * c32 >= kTinyExp) || (RES && __all((nd - md) * c32 >= kTinyExp))) dense |= 1u << u;
    if (!__any(vt >= tt || (RES && vd >= td))) continue;
#pragma unroll
    for (int e = 0; e < epv; ++e) {
      const bool l = xt[e] >= tt || (RES && xd[e] >= td);
      live |= (uint32_t)l << (u * epv + e);
    }
    __builtin_amdgcn_sched_barrier(0);  // one vector at a time (register pressure)
  }
  // fp32 triage of one token (bit `bit` of the lane's flags); a token of -inf
  // in both rows adds nothing and is not flagged
  const float rho32 = (float)J.rho;
  const float hi32 = (float)(J.rho * (1.0 + 2.0 * kRhoBand)), lo32 = (float)(J.rho * (1.0 - 2.0 * kRhoBand));
  auto triage = [&](float xt, float xd, int bit) {
    const float at = (xt - mt) * c32;
    const float et = exp2_f32(at);
    bool flag = at >= kTinyExp;
    // selects rather than branches: the sums take a term or +0
    if (RES) {
      const float ad = (xd - md) * c32;
      const float ed = exp2_f32(ad);
      flag |= ad >= kTinyExp;
      const bool pos = et > hi32 * ed;
      flag |= !pos && et > 0.f && et >= lo32 * ed;
      const bool take_pos = pos && !flag;
      st += flag ? 0.f : et;
      sd += flag ? 0.f : ed;
      sdp += take_pos ? et - rho32 * ed : 0.f;
      sbp += take_pos ? ed : 0.f;
    } else {
      st += flag ? 0.f : et;
    }
    flags |= (uint32_t)flag << bit;
  };
  if (!__any(__builtin_popcount(live) > kSparse)) {
    // few live tokens per lane (rows whose mass sits on a handful of tokens):
    // each is taken from the registers by its index and triaged alone
    uint32_t rest = live;
#pragma unroll 1
    while (__any(rest != 0u)) {
      const bool has = rest != 0u;
      const int i = has ? __builtin_ctz(rest) : 0;
      rest &= rest - 1u;
      float xt = token_at<DT>(wt[0], wt[1], wt[2], wt[3], i);
      float xd = RES ? token_at<DT>(wd[0], wd[1], wd[2], wd[3], i) : 0.f;
      if (!has) xt = xd = -INFINITY;
      triage(xt, xd, i);
    }
  } else {
    // fp32 triage of every token of the live vectors
#pragma unroll
    for (int u = 0; u < nv; ++u) {
      if ((dense >> u) & 1u) {
        flags |= ((1u << epv) - 1u) << (u * epv);
        continue;
      }
      if (!__any(((live >> (u * epv)) & ((1u << epv) - 1u)) != 0u)) continue;
      // unpacked again rather than kept from the mask pass (register pressure)
      uint4 t4 = wt[u], d4 = RES ? wd[u] : wt[u];
      __asm__ volatile("" : "+v"(t4.x), "+v"(t4.y), "+v"(t4.z), "+v"(t4.w));
      if (RES) __asm__ volatile("" : "+v"(d4.x), "+v"(d4.y), "+v"(d4.z), "+v"(d4.w));
      float xt[epv], xd[epv];
      unpack<DT>(t4, xt);
      if (RES) unpack<DT>(d4, xd);
#pragma unroll
      for (int e = 0; e < epv; ++e) triage(xt[e], RES ? xd[e] : 0.f, u * epv + e);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  ExactAcc A{(double)st, (double)sd, (double)sdp, (double)sbp, 0};
  // Nearly every token flagged (the busiest lane has at least 3/4 of its tokens
  // flagged; the flagged loop takes as many steps as that lane, each dearer than
  // a step of the straight pass): every token of the tile takes the straight
  // double-precision pass. The fp32 sums of the few unflagged tokens are then
  // dropped: double precision only makes their masses more accurate, and it
  // puts each on the side of the band its fp32 triage did (that side was clear
  // by twice the band).
  const int busiest = wave_minmax<true>(__builtin_popcount(flags));
  const bool all_flagged = busiest * 4 >= nv * epv * 3;
  if (all_flagged) A = ExactAcc{0.0, 0.0, 0.0, 0.0, 0};
  const bool any_flagged = __any(flags != 0u);
  if (any_flagged) {  // the fixups read the tile from an LDS copy
#pragma unroll
    for (int u = 0; u < nv; ++u) {
      G.t[wv][u][lane] = wt[u];
      if (RES) G.d[wv][u][lane] = wd[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
  }
  const Exp2Regs K = pinned_exp2();
  if (all_flagged) {
    // (nearly) every token of the tile is flagged (rows with mass everywhere):
    // the double-precision pass runs straight through the staged vectors,
    // token i of every lane at step i -- the order of the flagged loop below
    // when every token is flagged
    const double hi = J.rho * (1.0 + kRhoBand), lo = J.rho * (1.0 - kRhoBand);
    const unsigned long long below = (1ull << lane) - 1ull;
    // (no ballot between tokens, so that the tokens of a vector can overlap;
    // the undecided ones are appended afterwards, in the same order)
    uint32_t und = 0u;
#pragma unroll 1
    for (int u = 0; u < nv; ++u) {
      float xt[epv], xd[epv];
      unpack<DT>(G.t[wv][u][lane], xt);
      if (RES) unpack<DT>(G.d[wv][u][lane], xd);
#pragma unroll
      for (int e = 0; e < epv; ++e) {
        double et, ed;
        und |= (uint32_t)exact_sums<RES>(xt[e], RES ? xd[e] : 0.f, J, hi, lo, A, tab, K, et, ed) << (u * epv + e);
      }
    }
    if (RES) {
      // token i of every lane at step i, as the flagged loop orders them; the
      // masses again from the staged logits (the same arithmetic, the same values)
#pragma unroll 1
      while (__any(und != 0u)) {
        const int i = wave_minmax<false>(und != 0u ? __builtin_ctz(und) : 32);
        const bool mine = (und >> i) & 1u;
        und &= ~(1u << i);
        float xt = 0.f, xd = 0.f;
        double et = 0.0, ed = 0.0;
        if (mine) {
          xt = staged_at<DT>(G.t[wv][i / epv][lane], i % epv);
          xd = staged_at<DT>(G.d[wv][i / epv][lane], i % epv);
          et = emass_t(xt, J.mt, J.c64, tab, K);
          ed = emass_t(xd, J.md, J.c64, tab, K);
        }
        append_undecided<NW>(mine, xt, xd, et, ed, below, A, L, wv);
      }
    }
    __builtin_amdgcn_wave_barrier();
  } else if (any_flagged) {
    const double hi = J.rho * (1.0 + kRhoBand), lo = J.rho * (1.0 - kRhoBand);
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll 1
    while (__any(flags != 0u)) {
      const bool has = flags != 0u;
      const int i = has ? __builtin_ctz(flags) : 0;
      flags &= flags - 1u;
      float xt = 0.f, xd = 0.f;
      if (has) {
        xt = staged_at<DT>(G.t[wv][i / epv][lane], i % epv);
        if (RES) xd = staged_at<DT>(G.d[wv][i / epv][lane], i % epv);
      }
      exact_token<RES, NW>(has, xt, xd, J, hi, lo, below, A, L, wv, tab, K);
    }
    // the stage and the lists are reused by the wave's next tile
    __builtin_amdgcn_wave_barrier();
  }
  next();
  const double zt = wave_sum(A.zt);
  double zd = 0.0, dp = 0.0, bp = 0.0, gt = 0.0, gd = 0.0;  // lane g < ng holds group g's sums
  int ng = 0;
  if (RES) {
    zd = wave_sum(A.zd);
    dp = wave_sum(A.dp);
    bp = wave_sum(A.bp);
    const int n = A.n;
    if (n > kList) {
      ng = kRecOverflow;
    } else if (n > 0) {
      // the wave's list entries are complete before lanes read them
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      __builtin_amdgcn_wave_barrier();
      const bool have = lane < n;
      const double key = have ? L.dl[wv][lane] : 0.0;
      const double my_et = have ? L.et[wv][lane] : 0.0, my_ed = have ? L.ed[wv][lane] : 0.0;
      // first list entry with the same logit difference
      int first = lane;
      for (int e = 0; e < n; ++e) {
        const double ke = __shfl(key, e, 64);
        if (e < first && ke == key) first = e;
      }
      const unsigned long long leaders = __ballot(have && first == lane);
      ng = __builtin_popcountll(leaders);
      const int grp = __builtin_popcountll(leaders & ((1ull << first) - 1ull));
      if (ng > kGrp) {
        ng = kRecOverflow;
      } else {
        // group sums in list order: lane g accumulates the entries of group g
        for (int e = 0; e < n; ++e) {
          const int ge = __shfl(grp, e, 64);
          const double te = __shfl(my_et, e, 64), de = __shfl(my_ed, e, 64);
          if (lane == ge) { gt += te; gd += de; }
        }
      }
      // the lists are reused by the wave's next tile
      __builtin_amdgcn_wave_barrier();
    }
  }
  write_rec(rec, zt, zd, dp, bp, ng, gt, gd, lane);
}


// One wave's tiles k0, k0 + step, ... below ntile: a tile of a skipped chunk
// gets its record from the chunk's mass; the others take the tile pass.
template <int DT, bool RES, int NW>
__device__ __forceinline__ void wave_tiles(const char* trow, const char* drow, int V, int ntile, int k0, int step,
                                           const SampleJob& J, TileRec* R, const double* mass_t,
                                           const double* mass_d, TileSpace<NW>& TS, const double* tab, int wv,
                                           int lane) {
  constexpr int tok = TileTok<DT>::value;
  auto live = [&](int k) {  // the first tile from k on that is read, recording the skipped ones
    while (k < ntile && tile_skipped(J, k)) {
      const int ch = k / J.chunk_tiles;
      if (lane == 0) write_skipped_rec(R + k, k % J.chunk_tiles == 0, mass_t[ch], RES ? mass_d[ch] : 0.0);
      k += step;
    }
    return k;
  };
  auto load = [&](int k, uint4 (&t)[4], uint4 (&d)[4]) {
    load_tile_wave<DT>(trow, k * tok, V, lane, t);
    if (RES) load_tile_wave<DT>(drow, k * tok, V, lane, d);
  };
  // the next tile's loads are issued into the registers of the current one as
  // soon as its pass has finished with them (before its sums and record)
  int k = live(k0);
  if (k >= ntile) return;
  uint4 t[4], d[4];
  load(k, t, d);
#pragma unroll 1
  for (;;) {
    const int kn = live(k + step);
    tile_pass<DT, RES, NW>(t, d, J, R + k, TS, tab, wv, lane, [&] {
      if (kn < ntile) load(kn, t, d);
    });
    if (kn >= ntile) break;
    k = kn;
  }
}

// ---------------------------------------------------------------------------
// Pick.

// Fixed-order workgroup sum of doubles (same result in every thread).
template <int NW>
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = red[0];
  for (int w = 1; w < NW; ++w) t += red[w];
  __syncthreads();
  return t;
}

// A workgroup's tile: thread tid holds the bt contiguous tokens j0 + bt tid + i
// (-inf beyond V).
template <int DT, int NW>
__device__ __forceinline__ void load_tile_block(const char* rowp, int j0, int V, float* x) {
  constexpr int bt = TileGeom<DT, NW>::bt;
  constexpr int es = sizeof(typename Elem<DT>::T);
  const int jt = j0 + bt * (int)threadIdx.x;
  const char* p = rowp + (size_t)jt * es;
  if (bt * es == 16 && jt + bt <= V && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
    // the thread's tokens are one aligned 16-byte vector
    unpack<DT>(*reinterpret_cast<const uint4*>(p), x);
    return;
  }
#pragma unroll
  for (int i = 0; i < bt; ++i) {
    const int j = jt + i;
    x[i] = j < V ? Elem<DT>::at(rowp, j) : -INFINITY;
  }
}

// STAGED: the request's records are first copied into LDS (ntile <= kPickStage).
template <int DT, int NW, bool STAGED>
__device__ __forceinline__ void pick_impl(const char* trow, const char* drow, int V, int ntile, const SampleJob& J,
                                          TileRec* R, int32_t* dst, int force_exact, PickSpace<NW>& P,
                                          const double* tab) {
  constexpr int tok = TileGeom<DT, NW>::tok;
  constexpr int bt = TileGeom<DT, NW>::bt;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  // the records, copied into LDS in one pass when they fit
  constexpr bool staged = STAGED;
  if (staged) {
    const int nw = ntile * kRecWords;
    for (int e = tid; e < nw; e += NW * 64) P.rw[e] = rec_load(R + e / kRecWords, e % kRecWords);
    __syncthreads();
  }
  auto rw = [&](int k, int w) -> uint64_t { return staged ? P.rw[k * kRecWords + w] : rec_load(R + k, w); };
  auto rf = [&](int k, int w) -> double { return __longlong_as_double((long long)rw(k, w)); };
  auto rng = [&](int k) -> int { return (int)(uint32_t)rw(k, kRecNgrp); };
  // --- tile masses, total S, and the first tile whose inclusive prefix exceeds
  // u S (wave 0; rho = Z_t / Z_d for a residual)
  auto tile_mass = [&](int k, bool r, double rho) -> double {
    if (!r) return rf(k, kRecZt);
    const int ng = rng(k);
    if (ng == kRecRecomputed) return rf(k, kRecZd);
    double t = rf(k, kRecDpos) + (J.rho - rho) * rf(k, kRecBpos);
    for (int g = 0; g < ng; ++g) {
      const double q = rf(k, kRecGet + g) - rho * rf(k, kRecGed + g);
      t += q > 0.0 ? q : 0.0;
    }
    return t > 0.0 ? t : 0.0;
  };
  auto scan_tiles = [&](bool res, double rho) {
    // the tile masses, one per lane and 64-tile round, kept for the scan
    double part = 0.0;
    for (int k = lane; k < ntile; k += 64) part += tile_mass(k, res, rho);
    double S = wave_sum(part);
    if (!(S > 0.0) && res) {  // residual underflow: draw from p_t of the same row
      res = false;
      part = 0.0;
      for (int k = lane; k < ntile; k += 64) part += tile_mass(k, false, rho);
      S = wave_sum(part);
    }
    const double thr = (double)J.u * S;
    double base = 0.0;
    int tile = -1, lastpos = -1;
    double W = 0.0;
    for (int k0 = 0; k0 < ntile; k0 += 64) {
      const int k = k0 + lane;
      const double t = k < ntile ? tile_mass(k, res, rho) : 0.0;
      const double incl = wave_incl_scan(t);
      const unsigned long long pos = __ballot(t > 0.0);
      if (pos) lastpos = k0 + 63 - __builtin_clzll(pos);
      const unsigned long long hit = __ballot(t > 0.0 && base + incl > thr);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        tile = k0 + l;
        W = base + lane_f64(incl - t, l);
        break;
      }
      base += lane_f64(incl, 63);
    }
    if (lane == 0) {
      P.last_mode = tile < 0;  // rounding left no tile above u S: last token with positive mass
      P.tile = tile < 0 ? lastpos : tile;
      P.W = W;
      P.thr = thr;
      P.res = res;
    }
  };

  // --- exact normalisers (wave 0, lanes over tiles, fixed-order sums); the
  // scan follows in the same wave unless tiles must first be recomputed
  if (wv == 0) {
    double zt = 0.0, zd = 0.0;
    int need = 0;
    for (int k = lane; k < ntile; k += 64) {
      zt += rf(k, kRecZt);
      zd += rf(k, kRecZd);
      need |= rng(k) == kRecOverflow;
    }
    zt = wave_sum(zt);
    zd = wave_sum(zd);
    need = __any(need);
    const bool res = J.kind == JOB_RESIDUAL;
    const double rho = res ? zt / zd : 0.0;
    // every token outside the band has the same residual sign under rho and rho~
    const bool exact_all = res && (force_exact || !(fabs(rho - J.rho) <= 0.5 * kRhoBand * J.rho));
    const int any_exact = res && (exact_all || need) ? (exact_all ? 2 : 1) : 0;
    if (lane == 0) {
      P.Zt = zt;
      P.Zd = zd;
      P.any_exact = any_exact;
    }
    if (!any_exact) scan_tiles(res, rho);
  }
  __syncthreads();
  const double rho = J.kind == JOB_RESIDUAL ? P.Zt / P.Zd : 0.0;

  // --- tiles whose residual mass is recomputed token by token (then marked
  // kRecRecomputed, mass in zd), and the scan
  if (P.any_exact) {
    const bool all = P.any_exact == 2;
    const Exp2Regs K = pinned_exp2();
    for (int k = 0; k < ntile; ++k) {
      if (!(all || rng(k) == kRecOverflow)) continue;
      float xt[bt], xd[bt];
      load_tile_block<DT, NW>(trow, k * tok, V, xt);
      load_tile_block<DT, NW>(drow, k * tok, V, xd);
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < bt; ++i) {
        const double q = emass_t(xt[i], J.mt, J.c64, tab, K) - rho * emass_t(xd[i], J.md, J.c64, tab, K);
        acc += q > 0.0 ? q : 0.0;
      }
      acc = block_sum<NW>(acc, P.red);
      if (tid == 0) {
        if (staged) {
          P.rw[k * kRecWords + kRecZd] = f64_word(acc);
          P.rw[k * kRecWords + kRecNgrp] = ngrp_word(kRecRecomputed);
        } else {
          rec_store(R + k, kRecZd, f64_word(acc));
          rec_store(R + k, kRecNgrp, ngrp_word(kRecRecomputed));
        }
      }
      __builtin_amdgcn_s_waitcnt(0);  // the stores are complete before any wave reads them back
      __syncthreads();
    }
    if (wv == 0) scan_tiles(true, rho);
    __syncthreads();
  }
  const bool res = P.res != 0;
  const int tile = P.tile;
  if (tile < 0) {  // no positive mass anywhere (cannot happen for usable rows)
    if (tid == 0) *dst = -1;
    return;
  }
  const bool last_mode = P.last_mode != 0;
  const double thr = P.thr, Wtile = P.W;

  // --- masses of the chosen unit (a tile, or every tile of a skipped chunk), bt
  // contiguous tokens per thread, then a fixed-order scan from the unit's base
  int tile_end = tile + 1;
  if (!res && rng(tile) == kRecChunkHead) tile_end = min(ntile, tile + J.chunk_tiles);
  double base = Wtile;
  int found = 0x7fffffff, lastpos = -1;
  const Exp2Regs K = pinned_exp2();
  for (int t = tile; t < tile_end; ++t) {
    double q[bt];
    double local = 0.0;
    {
      float xt[bt], xd[bt];
      load_tile_block<DT, NW>(trow, t * tok, V, xt);
      if (res) load_tile_block<DT, NW>(drow, t * tok, V, xd);
#pragma unroll
      for (int i = 0; i < bt; ++i) {
        double v = emass_t(xt[i], J.mt, J.c64, tab, K);
        if (res) {
          v -= rho * emass_t(xd[i], J.md, J.c64, tab, K);
          v = v > 0.0 ? v : 0.0;
        }
        q[i] = v;
        local += v;
      }
    }
    const double wincl = wave_incl_scan(local);
    if (lane == 63) P.red[wv] = wincl;
    __syncthreads();
    double run = base;
    for (int w = 0; w < wv; ++w) run += P.red[w];
    run += wincl - local;
    double total = 0.0;  // the tile's sum, in the same order in every thread
    for (int w = 0; w < NW; ++w) total += P.red[w];
    const int jt = t * tok + tid * bt;
    int pk = 0x7fffffff, lp = -1;
#pragma unroll
    for (int i = 0; i < bt; ++i) {
      run += q[i];
      if (q[i] > 0.0) {
        lp = jt + i;
        if (!last_mode && run > thr && pk == 0x7fffffff) pk = jt + i;
      }
    }
    pk = wave_minmax<false>(pk);
    lp = wave_minmax<true>(lp);
    if (lane == 0) { P.smin[wv] = pk; P.smax[wv] = lp; }
    __syncthreads();
    for (int w = 0; w < NW; ++w) {
      found = min(found, P.smin[w]);
      lastpos = max(lastpos, P.smax[w]);
    }
    __syncthreads();  // P is reused by the next tile
    base = base + total;
    if (found != 0x7fffffff) break;
  }
  // no token passed u S in the unit (rounding at its end): the last positive token
  if (tid == 0) *dst = found != 0x7fffffff ? found : lastpos;
}

// The pick; STAGED (ntile <= kPickStage) copies the records into LDS first.
// Kernels are instantiated per variant, so that each keeps its own register
// allocation.
template <int DT, int NW, bool STAGED>
__device__ __forceinline__ void pick(const char* trow, const char* drow, int V, int ntile, const SampleJob& J, TileRec* R,
                     int32_t* dst, int force_exact, PickSpace<NW>& P, const double* tab) {
  pick_impl<DT, NW, STAGED>(trow, drow, V, ntile, J, R, dst, force_exact, P, tab);
}

}  // namespace sv
