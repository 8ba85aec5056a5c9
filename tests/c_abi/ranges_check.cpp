// Host check of the byte ranges the MXFP8 casts derive from their group tables
// (no GPU; built by tests/test_write_ranges.py with hipcc, host code only).
//
// It includes the casts' source, so it runs the very functions the kernels
// call to decode a work unit (dim1_unit, dim0_scale_row, dim0_zero_block) and
// to size the launch (dim1_geometry, dim0_geometry), with group tables built
// here on the host:
//   * a correct table (the kernels' scan written out plainly): every byte of
//     the blocked scale allocation is written exactly once (tiles, padding and
//     tail), every code (token, feature block) exactly once, and every read
//     and write lies inside its buffer;
//   * corrupted tables (every group width negated, as a miscompiled lane
//     shift once did; random values): every read and write still lies inside
//     its buffer.
// It also checks zero_share, fits and clamp_run on their own. Prints "ok" and
// exits 0 when every check holds.

#include "../../group_scale_factor_amd/csrc/mx_quantize.hip"

#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

namespace {

int failures = 0;
void fail(const std::string &what) {
  if (failures < 20) std::fprintf(stderr, "check failed: %s\n", what.c_str());
  ++failures;
}

// ---------------------------------------------------------------------------
// host group tables with the accessors the unit decoders use
// ---------------------------------------------------------------------------

// dim1: e = clamped cumulative end (scale columns), cch = cumulative tile
// columns, cw = cumulative padded widths.
struct Table1 {
  int groups = 0;
  std::vector<int> e, cch, cw;
  int count_cch_le(int64_t key) const {   // as the kernel's ballot: every group, in any order
    int n = 0;
    for (int g = 0; g < groups; ++g) n += int64_t(cch[g]) <= key;
    return n;
  }
  int end(int g) const { return e[g]; }
  int chunks_through(int g) const { return cch[g]; }
  int width_through(int g) const { return cw[g]; }
};

// The dim1 scan, written out: ends clamped into [0, T], to scale columns,
// running maximum; widths, padded widths, prefix sums. `sign` -1 negates every
// width (the corruption a reversed subtraction makes).
Table1 scan1(const Q1Params &p, const std::vector<int64_t> &offs, int sign) {
  Table1 t;
  t.groups = p.groups;
  int prev = 0, ch = 0, w = 0;
  for (int g = 0; g < p.groups; ++g) {
    int64_t et = p.group_tokens > 0 ? int64_t(g + 1) * p.group_tokens : offs[g];
    et = et < 0 ? 0 : (et > p.T ? p.T : et);
    const int e = std::max(int(et / 32), prev);
    const int width = sign * (e - prev);
    const int W = (width + 3) & ~3;
    ch += W / 4;
    w += W;
    t.e.push_back(e);
    t.cch.push_back(ch);
    t.cw.push_back(w);
    prev = e;
  }
  return t;
}

// dim0 (M groups): e = clamped cumulative end (rows), pend = padded cumulative end.
struct TableM {
  int groups = 0;
  std::vector<int> e, pend;
  int count_ends_le(int64_t key) const {
    int n = 0;
    for (int g = 0; g < groups; ++g) n += int64_t(e[g]) <= key;
    return n;
  }
  int count_pends_le(int64_t key) const {
    int n = 0;
    for (int g = 0; g < groups; ++g) n += int64_t(pend[g]) <= key;
    return n;
  }
  int end(int g) const { return e[g]; }
  int pend_at(int g) const { return pend[g]; }
};

TableM scanM(int rows, const std::vector<int64_t> &offs, int sign) {
  TableM t;
  t.groups = int(offs.size());
  int prev = 0, pend = 0;
  for (int64_t o : offs) {
    const int e = std::max(int(o < 0 ? 0 : (o > rows ? rows : o)), prev);
    pend += sign * ((e - prev + 127) / 128 * 128);
    t.e.push_back(e);
    t.pend.push_back(pend);
    prev = e;
  }
  return t;
}

template <class T>
void scramble(std::mt19937_64 &rng, std::vector<T> &v) {
  for (auto &x : v) x = T(int64_t(rng() % 200001) - 100000);
}

std::vector<int64_t> random_offsets(std::mt19937_64 &rng, int G, int64_t total, int64_t multiple) {
  std::vector<int64_t> o(G);
  for (auto &x : o) x = int64_t(rng() % uint64_t(total / multiple + 1)) * multiple;
  std::sort(o.begin(), o.end());
  if (rng() % 4) o[G - 1] = total;   // usually the groups cover everything
  if (rng() % 8 == 0) {               // sometimes offsets that break the order
    o[rng() % G] = int64_t(rng() % uint64_t(2 * total + 2)) - total / 2;
  }
  return o;
}

// ---------------------------------------------------------------------------
// dim1 cast
// ---------------------------------------------------------------------------

// Checks every unit of one launch, reached as the kernel reaches it (workgroup,
// then the half of a workgroup of two feature blocks, dim1_slot); every unit
// must be reached exactly once. `exact` adds the exactly-once coverage checks of
// the bytes written.
void check_dim1(const Q1Params &p, const Table1 &t, bool exact, const std::string &name) {
  const int64_t chunk_units = p.units / p.nb;
  const int blocks = dim1_blocks(p);
  std::vector<uint8_t> scale_hits(exact ? size_t(p.scale_bytes) : 0, 0);
  std::vector<uint8_t> token_hits(exact ? size_t(p.T / 32) * p.nb : 0, 0);
  std::vector<uint8_t> unit_hits(size_t(p.units), 0);
  const int64_t x_extent = p.group_tokens > 0 ? 0 : p.T * p.ld;   // elements
  if (p.wg_units * blocks < p.units || p.slots < p.wg_units) fail(name + ": fewer unit slots than units");
  for (int64_t wg = 0; wg < p.slots; ++wg) {
    for (int half = 0; half < blocks; ++half) {
      const Dim1Slot sl = dim1_slot(p, wg, blocks, half);
      if (sl.ci < 0 || sl.ci >= chunk_units || sl.fb < 0 || (sl.live && sl.fb >= p.nb)) {
        fail(name + ": workgroup slot outside the units");
        continue;
      }
      if (!sl.live) continue;
      ++unit_hits[size_t(sl.fb) * chunk_units + sl.ci];
      const int fb = sl.fb;
      const int64_t ci = sl.ci;
      const Dim1Unit un = dim1_unit(p, t, ci, fb);
      if (un.spare) {
        const ZeroSpan &z = un.zero;
        if (!(0 <= z.begin && z.begin <= z.full && z.full <= z.end && z.end <= p.scale_bytes &&
              (z.begin & 15) == 0 && ((z.end - z.full) & 3) == 0 && z.end - z.full < 16))
          fail(name + ": spare zero span outside the scale allocation");
        if (exact)
          for (int64_t b = z.begin; b < z.end; ++b) ++scale_hits[size_t(b)];
        continue;
      }
      if (un.ntok < 0 || un.ntok > 128 || un.ntok % 32 != 0) fail(name + ": token count");
      if (un.tile_off != -1 && !fits(un.tile_off, 512, p.scale_bytes)) fail(name + ": scale tile outside");
      if (un.ntok == 0) {
        // nothing read (a zero-size buffer) and no code written; the tile, if any, is counted below
      } else if (p.group_tokens > 0) {
        // expert g's input rows [0, K) at g * x_gstride, its codes: N rows of K bytes at g * q_gstride
        const int64_t g = un.t0 / p.group_tokens;
        const int64_t x0 = g * p.x_gstride, q0 = g * p.q_gstride;
        if (g < 0 || g >= p.groups) fail(name + ": expert index");
        if (un.x_row0 < x0 || un.x_row0 + int64_t(un.ntok) * p.ld > x0 + int64_t(p.group_tokens) * p.ld)
          fail(name + ": expert input rows outside");
        if (un.q_col0 < q0 || un.q_col0 + un.ntok > q0 + p.group_tokens) fail(name + ": expert code columns outside");
      } else {
        if (un.t0 < 0 || un.t0 + un.ntok > p.T) fail(name + ": token run outside [0, T)");
        if (un.x_row0 < 0 || un.x_row0 + int64_t(un.ntok) * p.ld > x_extent) fail(name + ": input rows outside");
        if (un.q_col0 < 0 || un.q_col0 + un.ntok > p.q_ld) fail(name + ": code columns outside");
      }
      if (exact) {
        if (un.tile_off >= 0)
          for (int64_t b = un.tile_off; b < un.tile_off + 512; ++b) ++scale_hits[size_t(b)];
        for (int64_t k = 0; k < un.ntok / 32; ++k) ++token_hits[size_t(fb) * (p.T / 32) + un.t0 / 32 + k];
      }
    }
  }
  for (size_t k = 0; k < unit_hits.size(); ++k)
    if (unit_hits[k] != 1) {
      fail(name + ": unit " + std::to_string(k) + " reached " + std::to_string(unit_hits[k]) + " times");
      break;
    }
  if (exact) {
    for (int64_t b = 0; b < p.scale_bytes; ++b)
      if (scale_hits[size_t(b)] != 1) {
        fail(name + ": scale byte " + std::to_string(b) + " written " + std::to_string(scale_hits[size_t(b)]) +
             " times");
        break;
      }
    for (size_t k = 0; k < token_hits.size(); ++k)
      if (token_hits[k] != 1) {
        fail(name + ": token block " + std::to_string(k) + " coded " + std::to_string(token_hits[k]) + " times");
        break;
      }
  }
}

void dim1_cases(std::mt19937_64 &rng) {
  for (int it = 0; it < 2000; ++it) {
    const bool experts = it % 4 == 3;
    Q1Params p = {};
    int64_t N = 1 + int64_t(rng() % 300);
    std::vector<int64_t> offs;
    if (experts) {
      const int E = 1 + int(rng() % 6);
      const int64_t K = 32 * int64_t(1 + rng() % 12);
      p.T = E * K;
      p.q_ld = K;
      p.group_tokens = int(K);
      p.groups = E;
      p.ld = N + 8 * int64_t(rng() % 3);
      p.x_gstride = K * p.ld + 8 * int64_t(rng() % 4);
      p.q_gstride = N * K;
      // the entry point's rule (K a multiple of 128), and every other case too
      p.diagonal = K % 128 == 0 || (it / 4) % 2 == 1;
      p.scale_bytes = mx_quantize_dim1_3d_scale_bytes(E, K, N);
    } else {
      p.T = 32 * int64_t(rng() % 40);
      p.q_ld = p.T;
      p.groups = 1 + int(rng() % (it % 5 == 0 ? 70 : 6));
      p.ld = N + 8 * int64_t(rng() % 3);
      offs = random_offsets(rng, p.groups, p.T, rng() % 2 ? 32 : 1);
      p.scale_bytes = mx_quantize_dim1_K_groups_scale_bytes(p.T, N, p.groups);
    }
    if (p.scale_bytes <= 0) continue;
    if (!dim1_geometry(p, N)) {
      fail("dim1 geometry rejected a small shape");
      continue;
    }
    // every third case in runs of workgroups dealt to the XCDs in turn (the order of large launches),
    // with the launch's run length or a random one
    if (it % 3 == 1) {
      p.deal = it % 2 ? kDim1DealUnits : 1 + int64_t(rng() % 20);
      p.slots = slots_for(true, p.wg_units, p.deal);
    }
    const std::string name = "dim1 case " + std::to_string(it) + (p.deal ? " (runs)" : "");
    // the correct table: exact coverage (offsets that break the order are clamped by the scan)
    check_dim1(p, scan1(p, offs, 1), true, name);
    // corrupted tables: bounds only
    check_dim1(p, scan1(p, offs, -1), false, name + " (negated widths)");
    Table1 t = scan1(p, offs, 1);
    scramble(rng, t.e);
    scramble(rng, t.cch);
    scramble(rng, t.cw);
    check_dim1(p, t, false, name + " (random table)");
  }
}

// ---------------------------------------------------------------------------
// dim0 cast
// ---------------------------------------------------------------------------

void check_dim0(const QParams &p, const TableM &t, bool exact, const std::string &name) {
  std::vector<uint8_t> hits(exact ? size_t(p.scale_bytes) : 0, 0);
  auto word = [&](int64_t off) {
    // the kernel stores a word only where fits() allows it
    if (!fits(off, 4, p.scale_bytes)) {
      if (exact) fail(name + ": a correct table placed a scale word outside the allocation");
      return;
    }
    if (exact)
      for (int k = 0; k < 4; ++k) ++hits[size_t(off + k)];
  };
  for (int64_t r = 0; r < p.rows; ++r) {
    const int64_t R = dim0_scale_row(t, p.groups, r);
    if (R >= 0)
      for (int tc = 0; tc < p.tile_cols; ++tc) word(scale_word_offset(R, tc, p.tile_cols));
  }
  for (int64_t ob = 0; ob < p.pad_blocks; ++ob) {
    const Dim0ZeroBlock z = dim0_zero_block(p, t, ob);
    if (z.in_group) {
      if (z.valid < 0 || z.valid > kTileRows) fail(name + ": padding rows of a block");
      for (int rr = z.valid; rr < kTileRows; ++rr)
        for (int tc = 0; tc < p.tile_cols; ++tc) word(scale_word_offset(ob * kTileRows + rr, tc, p.tile_cols));
    } else {
      const ZeroSpan &s = z.tail;
      if (!(0 <= s.begin && s.begin <= s.full && s.full <= s.end && s.end <= p.scale_bytes && (s.begin & 15) == 0))
        fail(name + ": tail zero span outside the scale allocation");
      if (exact)
        for (int64_t b = s.begin; b < s.end; ++b) ++hits[size_t(b)];
    }
  }
  if (exact)
    for (int64_t b = 0; b < p.scale_bytes; ++b)
      if (hits[size_t(b)] != 1) {
        fail(name + ": scale byte " + std::to_string(b) + " written " + std::to_string(hits[size_t(b)]) + " times");
        break;
      }
}

void dim0_cases(std::mt19937_64 &rng) {
  for (int it = 0; it < 2000; ++it) {
    const int64_t rows = int64_t(rng() % 1200);
    const int64_t K = 32 * int64_t(1 + rng() % 24);
    const int G = 1 + int(rng() % (it % 5 == 0 ? 70 : 6));
    QParams p = {};
    dim0_geometry(p, rows, K, G);
    if (p.scale_bytes <= 0) continue;
    const std::vector<int64_t> offs = random_offsets(rng, G, rows, 1);
    const std::string name = "dim0 case " + std::to_string(it);
    check_dim0(p, scanM(int(rows), offs, 1), true, name);
    check_dim0(p, scanM(int(rows), offs, -1), false, name + " (negated sizes)");
    TableM t = scanM(int(rows), offs, 1);
    scramble(rng, t.e);
    scramble(rng, t.pend);
    check_dim0(p, t, false, name + " (random table)");
  }
}

// ---------------------------------------------------------------------------
// the clamps on their own
// ---------------------------------------------------------------------------

void clamp_cases(std::mt19937_64 &rng) {
  // zero_share: the parts tile the clamped range exactly, in order, 16-byte aligned starts
  for (int it = 0; it < 20000; ++it) {
    const int64_t limit = 4 * int64_t(rng() % 300);
    const int64_t lo = int64_t(rng() % 1400) - 300, hi = int64_t(rng() % 1400) - 300;
    const int64_t parts = int64_t(rng() % 9);
    const int64_t clo = std::min(std::max(lo, int64_t(0)), limit) & ~int64_t(15);
    const int64_t chi = std::max(clo, std::min(hi, limit)) & ~int64_t(3);
    int64_t next = clo;
    for (int64_t part = -1; part <= parts; ++part) {
      const ZeroSpan z = zero_share(lo, hi, limit, part, parts);
      if (part < 0 || part >= parts) {
        if (z.begin != z.end) fail("zero_share: a part outside [0, parts) got bytes");
        continue;
      }
      if (z.begin == z.end) continue;
      if (z.begin != next || (z.begin & 15) || z.full < z.begin || z.end < z.full || z.end - z.full >= 16 ||
          ((z.full - z.begin) & 15) || z.end > limit || z.begin < 0)
        fail("zero_share: part " + std::to_string(part) + " of [" + std::to_string(lo) + ", " + std::to_string(hi) +
             ") in " + std::to_string(limit));
      next = z.end;
    }
    if (parts > 0 && chi > clo && next != chi) fail("zero_share: parts do not cover the clamped range");
  }
  // clamp_run and fits
  for (int it = 0; it < 20000; ++it) {
    const int64_t limit = int64_t(rng() % 200) - 20, first = int64_t(rng() % 400) - 200, n = int64_t(rng() % 400) - 200;
    const Run r = clamp_run(first, n, limit);
    const int64_t lim = limit < 0 ? 0 : limit;
    if (r.first < 0 || r.first > lim || r.n < 0 || r.first + r.n > lim) fail("clamp_run outside");
    if (first >= 0 && n >= 0 && first + n <= lim && (r.first != first || r.n != n)) fail("clamp_run moved a valid run");
    const bool f = fits(first, n, limit);
    if (f != (n >= 0 && first >= 0 && first + n <= limit)) fail("fits");
  }
}

}  // namespace

int main() {
  std::mt19937_64 rng(20261203);
  clamp_cases(rng);
  dim1_cases(rng);
  dim0_cases(rng);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
