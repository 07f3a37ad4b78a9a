// Host-side check of the kernels' LDS tile index math, compiled from the
// same header the kernels use (io_aware_tiled_attn_amd/csrc/fa_layout.h).
// Test infrastructure: built into tests/_build/liblayout_check.so and called
// from tests/test_pipeline_model.py; no kernel runs here.
//
// For every tile shape the kernels accept (and the wider shapes that were
// tried and set aside), it checks
//   * the global -> LDS copies: every LDS chunk of a tile is written once,
//     every (row, chunk) of the tile's rows is fetched once, and no row lies
//     outside the tile;
//   * every MFMA operand read: in bounds, aligned, and returning the row
//     and column the operand layout asks for once the chunk permutation the
//     copies applied is undone;
//   * the bank spread of each read instruction (the LDS serves 256 bytes a
//     cycle: 16 lanes of a 16-byte read or 32 lanes of an 8-byte read); the
//     degree (1 = conflict-free) is reported, and for the backward's tiles,
//     designed conflict-free, a degree above 1 counts as a violation;
//   * the forward's Q staging slots (apart from each other and from the
//     tiles copied meanwhile) and the LDS each launch reserves against the
//     160 KB of a CU;
//   * the forward epilogue's output staging: every output element written
//     once and read back by the lane that stores its row, each store
//     instruction covering 1 KB of consecutive rows;
//   * the forward's workgroup order: every (head, query tile) exactly once,
//     each head on one XCD, each head group heaviest tile first, and group
//     sizes that divide the XCD's heads and fit what it runs at once.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../io_aware_tiled_attn_amd/csrc/fa_layout.h"

namespace {

using namespace fa::layout;

struct Report {
  int violations = 0;
  std::string text;
  void note(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    text += buf;
    text += "\n";
  }
  void fail(const char* fmt, ...) {
    ++violations;
    if (violations > 40) return;   // enough to diagnose
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    text += "VIOLATION ";
    text += buf;
    text += "\n";
  }
};

// A tile whose rows are row_bytes wide, written by copy instructions with
// the permutation f.  Records which (row, chunk) each LDS chunk holds.
template <typename F>
struct Tile {
  int rows, row_bytes, bytes;
  F f;
  std::vector<int> holder;   // per LDS chunk: row * chunks + chunk, or -1
  Tile(int rows_, int row_bytes_, F f_) : rows(rows_), row_bytes(row_bytes_), bytes(rows_ * row_bytes_), f(f_) {}

  // Run the copies: n_inst instructions of 64 lanes.
  void copy(Report& rep, const char* what) {
    const int cpr = row_bytes / 16;
    holder.assign(bytes / 16, -1);
    std::vector<int> fetched(rows * cpr, 0);
    if (bytes % 1024 != 0) rep.fail("%s: tile of %d bytes is not whole 1 KB copies", what, bytes);
    for (int inst = 0; inst < bytes / 1024; ++inst)
      for (int lane = 0; lane < 64; ++lane) {
        int row, chunk;
        copy_slot(row_bytes, inst, lane, f, row, chunk);
        const int dst = inst * 1024 + 16 * lane;
        if (row < 0 || row >= rows || chunk < 0 || chunk >= cpr) {
          rep.fail("%s: copy inst %d lane %d fetches row %d chunk %d outside the tile", what, inst, lane, row, chunk);
          continue;
        }
        if (dst + 16 > bytes) rep.fail("%s: copy inst %d lane %d writes byte %d past the tile", what, inst, lane, dst);
        // The permutation must put this chunk where the copy writes it.
        if (dst != row * row_bytes + 16 * (chunk ^ f(row)))
          rep.fail("%s: copy inst %d lane %d writes (row %d, chunk %d) to byte %d, the layout puts it at %d", what,
                   inst, lane, row, chunk, dst, row * row_bytes + 16 * (chunk ^ f(row)));
        if (holder[dst / 16] != -1) rep.fail("%s: LDS chunk %d written twice", what, dst / 16);
        holder[dst / 16] = row * cpr + chunk;
        fetched[row * cpr + chunk]++;
      }
    for (int i = 0; i < rows * cpr; ++i)
      if (fetched[i] != 1) rep.fail("%s: (row %d, chunk %d) fetched %d times", what, i / cpr, i % cpr, fetched[i]);
  }

  // The element a read of `width` bytes at `byte` returns: checks bounds and
  // alignment, then compares the (row, chunk, byte in chunk) that LDS chunk
  // holds with the expected one.
  void expect(Report& rep, const char* what, int byte, int width, int row, int chunk, int within) {
    if (byte < 0 || byte + width > bytes) {
      rep.fail("%s: read of %d bytes at %d outside the %d-byte tile", what, width, byte, bytes);
      return;
    }
    if (byte % width != 0) rep.fail("%s: read of %d bytes at %d misaligned", what, width, byte);
    const int cpr = row_bytes / 16;
    const int h = holder[byte / 16];
    if (h != row * cpr + chunk || byte % 16 != within)
      rep.fail("%s: read at byte %d returns (row %d, chunk %d, +%d), wanted (row %d, chunk %d, +%d)", what, byte,
               h / cpr, h % cpr, byte % 16, row, chunk, within);
  }
};

template <typename F>
Tile<F> make_tile(int rows, int row_bytes, F f) {
  return Tile<F>(rows, row_bytes, f);
}

// Conflict degree of one read instruction: the LDS serves 256 bytes (64
// banks of 4 bytes) per cycle, `per` lanes at a time; the degree is the
// largest number of distinct words any bank must deliver in one group.
int conflict_degree(const std::vector<int>& byte_of_lane, int width) {
  const int per = 256 / width;
  int worst = 1;
  for (int g0 = 0; g0 < 64; g0 += per) {
    std::vector<std::vector<int>> words(64);
    for (int l = g0; l < g0 + per; ++l)
      for (int w = 0; w < width / 4; ++w) {
        const int word = byte_of_lane[l] / 4 + w;
        auto& v = words[word % 64];
        bool seen = false;
        for (int x : v) seen |= x == word;
        if (!seen) v.push_back(word);
      }
    for (auto& v : words)
      if ((int)v.size() > worst) worst = (int)v.size();
  }
  return worst;
}

// ---------------------------------------------------------------------------
// bf16 forward, tiles of BN keys x D.
// ---------------------------------------------------------------------------
template <int D, int BN>
void check_fwd(Report& rep, bool launched) {
  char what[96];
  using Z = FwdSwizzle<D>;
  auto kf = [](int r) { return Z::k(r); };
  auto vf = [](int r) { return Z::v(r); };
  auto K = make_tile(BN, 2 * D, kf);
  auto V = make_tile(BN, 2 * D, vf);
  snprintf(what, sizeof what, "fwd bf16 D=%d BN=%d K copy", D, BN);
  K.copy(rep, what);
  snprintf(what, sizeof what, "fwd bf16 D=%d BN=%d V copy", D, BN);
  V.copy(rep, what);
  if ((BN * D * 2) % 4096 != 0) rep.fail("fwd bf16 D=%d BN=%d: a tile does not split over four waves", D, BN);
  int kdeg = 1, vdeg = 1;
  // K as the A operand of S^T = K Q^T: lane (lc, lg), k-step ks, 32-key block mb.
  for (int ks = 0; ks < D / 16; ++ks)
    for (int mb = 0; mb < BN / 32; ++mb) {
      std::vector<int> at(64);
      for (int lane = 0; lane < 64; ++lane) {
        const int lc = lane & 31, lg = lane >> 5;
        at[lane] = 2 * (fwd_koff<D>(lc, lg, ks) + 32 * mb * D);
        snprintf(what, sizeof what, "fwd bf16 D=%d BN=%d K read ks=%d mb=%d lane=%d", D, BN, ks, mb, lane);
        K.expect(rep, what, at[lane], 16, 32 * mb + lc, 2 * ks + lg, 0);
      }
      const int d = conflict_degree(at, 16);
      if (d > kdeg) kdeg = d;
    }
  // V^T as the A operand of O^T += V^T P^T: per 16-key step c the two
  // transposing reads at rows 16 c and 16 c + 8.
  for (int dm = 0; dm < D / 32; ++dm)
    for (int c = 0; c < BN / 16; ++c)
      for (int h = 0; h < 16; h += 8) {
        std::vector<int> at(64);
        for (int lane = 0; lane < 64; ++lane) {
          const int sl = lane & 15, G = (lane >> 4) & 1, g = lane >> 5;
          at[lane] = 2 * (fwd_voff<D>(lane, dm) + (16 * c + h) * D);
          snprintf(what, sizeof what, "fwd bf16 D=%d BN=%d V read dm=%d c=%d h=%d lane=%d", D, BN, dm, c, h, lane);
          V.expect(rep, what, at[lane], 8, 16 * c + h + 4 * g + (sl >> 2), 4 * dm + 2 * G + ((sl & 3) >> 1),
                   8 * (sl & 1));
        }
        const int d = conflict_degree(at, 8);
        if (d > vdeg) vdeg = d;
      }
  // Q staging slots (prologue): each wave's 32 x D slot lies in the third K
  // or V buffer or past the six buffers, apart from the other slots and
  // from tiles 0 and 1, which are copied while Q is read.
  const int kTile = BN * D, slot = 32 * D, qend = 6 * kTile + fwd_qslot_extra<D, BN>();
  for (int w = 0; w < 8; ++w) {
    const int a = fwd_qslot<D, BN>(w);
    if (a < 0 || a + slot > qend) rep.fail("fwd bf16 D=%d BN=%d: Q slot of wave %d outside [0, %d)", D, BN, w, qend);
    for (int u = 0; u < w; ++u) {
      const int b = fwd_qslot<D, BN>(u);
      if (a < b + slot && b < a + slot) rep.fail("fwd bf16 D=%d BN=%d: Q slots of waves %d and %d overlap", D, BN, u, w);
    }
    for (int buf : {0, 1, 3, 4})
      if (a < (buf + 1) * kTile && buf * kTile < a + slot)
        rep.fail("fwd bf16 D=%d BN=%d: Q slot of wave %d overlaps tile buffer %d", D, BN, w, buf);
  }
  // LDS of a launch: three K and three V buffers, the Q slots past them,
  // then the sparse tile list (sparse launches use 32- and 64-key tiles; at
  // most N / BN + 1 ints, N <= 65536 keeps it within 8 KB); at least the
  // output staging of the epilogue (8 waves x 32 x D).
  const int list = 128 % BN == 0 ? 4 * (65536 / BN + 1) : 0;
  const int staged = 8 * 32 * D * 2;
  const int lds = 2 * qend + list > staged ? 2 * qend + list : staged;
  const bool fits = lds <= 160 * 1024;
  if (launched && !fits)
    rep.fail("fwd bf16 D=%d BN=%d: %d bytes of tiles, Q slots and the tile list exceed 160 KB", D, BN, lds);
  rep.note("fwd bf16 D=%d BN=%d (%s): LDS %d B%s, K read conflict degree %d, V read degree %d", D, BN,
           launched ? "launched" : "not launched", lds, fits ? "" : " (over 160 KB)", kdeg, vdeg);
}

// ---------------------------------------------------------------------------
// FP8 forward, tiles of BN keys x D bytes.
// ---------------------------------------------------------------------------
template <int D, int BN>
void check_fp8(Report& rep, bool launched) {
  char what[96];
  using Z = Fp8Swizzle<D>;
  auto kf = [](int r) { return Z::k(r); };
  auto vf = [](int r) { return Z::v(r); };
  auto K = make_tile(BN, D, kf);
  auto V = make_tile(BN, D, vf);
  snprintf(what, sizeof what, "fwd fp8 D=%d BN=%d K copy", D, BN);
  K.copy(rep, what);
  snprintf(what, sizeof what, "fwd fp8 D=%d BN=%d V copy", D, BN);
  V.copy(rep, what);
  if ((BN * D) % 4096 != 0) rep.fail("fwd fp8 D=%d BN=%d: a tile does not split over four waves", D, BN);
  // The 32 S^T rows of a block must hold 32 distinct keys of the block.
  {
    int seen = 0;
    for (int rho = 0; rho < 32; ++rho) seen |= 1 << fp8_kperm(rho);
    if (seen != -1) rep.fail("fp8 key order of S^T rows is not a permutation of 32 keys");
  }
  int kdeg = 1, vdeg = 1;
  for (int ks = 0; ks < D / 64; ++ks)
    for (int p = 0; p < 2; ++p)
      for (int mb = 0; mb < BN / 32; ++mb) {
        std::vector<int> at(64);
        for (int lane = 0; lane < 64; ++lane) {
          const int lc = lane & 31, lg = lane >> 5;
          at[lane] = fp8_koff<D>(lc, lg, ks, p) + 32 * mb * D;
          snprintf(what, sizeof what, "fwd fp8 D=%d BN=%d K read ks=%d p=%d mb=%d lane=%d", D, BN, ks, p, mb, lane);
          K.expect(rep, what, at[lane], 16, 32 * mb + fp8_kperm(lc), 4 * ks + 2 * lg + p, 0);
        }
        const int d = conflict_degree(at, 16);
        if (d > kdeg) kdeg = d;
      }
  // V^T operand of a 64-key step j: four transposing reads, 0, 8, 32 and 40
  // rows below the lane's first row.
  const int extra[4] = {0, 8, 32, 40};
  for (int dm = 0; dm < D / 32; ++dm)
    for (int j = 0; j < BN / 64; ++j)
      for (int e = 0; e < 4; ++e) {
        std::vector<int> at(64);
        for (int lane = 0; lane < 64; ++lane) {
          const int sl = lane & 15, G = (lane >> 4) & 1, g = lane >> 5;
          at[lane] = fp8_voff<D>(lane, dm) + (64 * j + extra[e]) * D;
          snprintf(what, sizeof what, "fwd fp8 D=%d BN=%d V read dm=%d j=%d e=%d lane=%d", D, BN, dm, j, e, lane);
          V.expect(rep, what, at[lane], 8, 64 * j + extra[e] + 16 * g + (sl >> 1), 2 * dm + G, 8 * (sl & 1));
        }
        const int d = conflict_degree(at, 8);
        if (d > vdeg) vdeg = d;
      }
  // Three K and three V tiles; after the loop the same LDS stages each
  // wave's 32 output rows (bf16): 8 waves at d = 64, 12 (three groups) at
  // d = 128.
  const int tiles = 2 * 3 * BN * D, stage = (D == 128 ? 12 : 8) * 32 * D * 2;
  const int lds = tiles > stage ? tiles : stage;
  if (lds > 160 * 1024) rep.fail("fwd fp8 D=%d BN=%d: %d bytes of tiles or staging exceed 160 KB", D, BN, lds);
  rep.note("fwd fp8 D=%d BN=%d (%s): LDS %d B, K read conflict degree %d, V read degree %d", D, BN,
           launched ? "launched" : "not launched", lds, kdeg, vdeg);
}

// ---------------------------------------------------------------------------
// Backward, fp16 tiles of D columns: 128 resident rows, 32-row blocks.  The
// kernels read with byte addresses built as (lane constant) XOR (32 ks) for
// rows and (lane constant) XOR (64 dm) + 32 c D for columns; both forms are
// checked against the plain formulas and the copies.
// ---------------------------------------------------------------------------
template <int D>
void check_bwd(Report& rep, int rows) {
  char what[96];
  auto f = [](int r) { return bwd_swz<D>(r); };
  auto T = make_tile(rows, 2 * D, f);
  snprintf(what, sizeof what, "bwd D=%d rows=%d copy", D, rows);
  T.copy(rep, what);
  int rdeg = 1, tdeg = 1;
  for (int rb = 0; rb < rows; rb += 32)
    for (int ks = 0; ks < D / 16; ++ks) {
      std::vector<int> at(64);
      for (int lane = 0; lane < 64; ++lane) {
        const int lc = lane & 31, lg = lane >> 5;
        const int fast = (int)((2u * (unsigned)bwd_chunk_off<D>(lc, lg)) ^ (32u * ks)) + 2 * rb * D;
        at[lane] = 2 * bwd_chunk_off<D>(rb + lc, 2 * ks + lg);
        if (fast != at[lane])
          rep.fail("bwd D=%d row read rb=%d ks=%d lane=%d: XOR address %d != %d", D, rb, ks, lane, fast, at[lane]);
        snprintf(what, sizeof what, "bwd D=%d rows=%d row read rb=%d ks=%d lane=%d", D, rows, rb, ks, lane);
        T.expect(rep, what, at[lane], 16, rb + lc, 2 * ks + lg, 0);
      }
      const int d = conflict_degree(at, 16);
      if (d > rdeg) rdeg = d;
    }
  for (int r16 = 0; r16 < rows; r16 += 16)
    for (int h = 0; h < 16; h += 8)
      for (int dm = 0; dm < D / 32; ++dm) {
        std::vector<int> at(64);
        for (int lane = 0; lane < 64; ++lane) {
          const int s = lane & 15, G = (lane >> 4) & 1, g = lane >> 5;
          const unsigned lc0 = 2u * (unsigned)bwd_tr_off<D>(lane, h, 0);
          const int fast = (int)((lc0 ^ (64u * dm)) + 32u * (unsigned)(r16 / 16) * D);
          at[lane] = 2 * bwd_tr_off<D>(lane, r16 + h, dm);
          if (fast != at[lane])
            rep.fail("bwd D=%d column read r=%d h=%d dm=%d lane=%d: XOR address %d != %d", D, r16, h, dm, lane, fast,
                     at[lane]);
          snprintf(what, sizeof what, "bwd D=%d rows=%d column read r=%d h=%d dm=%d lane=%d", D, rows, r16, h, dm,
                   lane);
          T.expect(rep, what, at[lane], 8, r16 + h + 4 * g + (s >> 2), 4 * dm + 2 * G + ((s & 3) >> 1), 8 * (s & 1));
        }
        const int d = conflict_degree(at, 8);
        if (d > tdeg) tdeg = d;
      }
  if (rdeg > 1 || tdeg > 1)
    rep.fail("bwd D=%d rows=%d: bank conflicts (row reads %d, column reads %d)", D, rows, rdeg, tdeg);
  rep.note("bwd D=%d rows=%d: row read conflict degree %d, column read degree %d", D, rows, rdeg, tdeg);
}

// LDS the backward launches reserve: dK/dV kernel (resident K, V; two
// buffers of Q, dO and row terms per group; or the closing sum) and dQ
// kernel (three K, V buffers per group and the Q/dO slots past them; or its
// closing sum), each plus the sparse block list (at most N / 32 + 1 ints,
// N <= 65536).
template <int D>
void check_bwd_lds(Report& rep) {
  const int res = 2 * 128 * D * 2, stage = 2 * 32 * D * 2 + 32 * 8, red = D * 4 * 64 * 4;
  const int dkdv = (res + 4 * stage > red ? res + 4 * stage : red) + 4 * (65536 / 32 + 1);
  const int dq = (8 * 2 * 32 * D * 2 > red / 2 ? 8 * 2 * 32 * D * 2 : red / 2) + 4 * (65536 / 32 + 1);
  if (dkdv > 160 * 1024) rep.fail("bwd D=%d: dK/dV kernel LDS %d B exceeds 160 KB", D, dkdv);
  if (dq > 160 * 1024) rep.fail("bwd D=%d: dQ kernel LDS %d B exceeds 160 KB", D, dq);
  rep.note("bwd D=%d: LDS at most %d B (dK/dV), %d B (dQ)", D, dkdv, dq);
}

// Output staging of the forward epilogue (bf16 and FP8 kernels): each lane's
// 8-byte writes of its query's features, then the 1 KB read-back whose lanes
// store whole consecutive rows to global memory.
template <int D>
void check_ostage(Report& rep) {
  const int row_bytes = 2 * D, bytes = 32 * row_bytes;
  std::vector<int> owner(bytes / 8, -1);   // per 8-byte slot: row * (D / 4) + 4-feature group
  std::vector<int> wbyte(64);
  int wdeg = 1;
  for (int dm = 0; dm < D / 32; ++dm)
    for (int i = 0; i < 4; ++i) {
      for (int lane = 0; lane < 64; ++lane) {
        const int lc = lane & 31, lg = lane >> 5;
        const int b = 2 * fwd_ostage_off<D>(lc, lg, dm, i);
        wbyte[lane] = b;
        if (b < 0 || b + 8 > bytes || b % 8 != 0) {
          rep.fail("ostage D=%d: write at byte %d outside or misaligned", D, b);
          continue;
        }
        if (owner[b / 8] != -1) rep.fail("ostage D=%d: byte %d written twice", D, b);
        owner[b / 8] = lc * (D / 4) + (32 * dm + 8 * i + 4 * lg) / 4;
      }
      const int d = conflict_degree(wbyte, 8);
      if (d > wdeg) wdeg = d;
    }
  for (size_t k = 0; k < owner.size(); ++k)
    if (owner[k] == -1) rep.fail("ostage D=%d: slot %zu never written", D, k);
  std::vector<int> rbyte(64), seen(32 * (D / 8), 0);
  int rdeg = 1;
  for (int inst = 0; inst < bytes / 1024; ++inst) {
    int lo = 1 << 30, hi = -1;
    for (int lane = 0; lane < 64; ++lane) {
      int row, chunk;
      copy_slot(row_bytes, inst, lane, FwdSwizzle<D>::k, row, chunk);
      const int b = inst * 1024 + 16 * lane;
      rbyte[lane] = b;
      if (row < 0 || row >= 32 || chunk < 0 || chunk >= D / 8) {
        rep.fail("ostage D=%d: read inst %d lane %d names row %d chunk %d", D, inst, lane, row, chunk);
        continue;
      }
      // The 16 bytes read must be features 8 chunk .. 8 chunk + 7 of `row`.
      if (owner[b / 8] != row * (D / 4) + 2 * chunk || owner[b / 8 + 1] != row * (D / 4) + 2 * chunk + 1)
        rep.fail("ostage D=%d: read inst %d lane %d gets slots (%d, %d), wanted row %d chunk %d", D, inst, lane,
                 owner[b / 8], owner[b / 8 + 1], row, chunk);
      seen[row * (D / 8) + chunk]++;
      const int g = row * row_bytes + 16 * chunk;   // global byte offset within the wave's rows
      lo = g < lo ? g : lo;
      hi = g + 16 > hi ? g + 16 : hi;
    }
    if (lo != inst * 1024 || hi != inst * 1024 + 1024)
      rep.fail("ostage D=%d: store inst %d covers global bytes [%d, %d), not one whole 1 KB", D, inst, lo, hi);
    const int d = conflict_degree(rbyte, 16);
    if (d > rdeg) rdeg = d;
  }
  for (size_t k = 0; k < seen.size(); ++k)
    if (seen[k] != 1) rep.fail("ostage D=%d: (row, chunk) %zu read %d times", D, k, seen[k]);
  if (rdeg > 1) rep.fail("ostage D=%d: read-back conflict degree %d", D, rdeg);
  rep.note("ostage D=%d: write conflict degree %d, read-back degree %d", D, wdeg, rdeg);
}

// Workgroup order of the forward launches (xcd_head_groups with the group
// size head_group_size picks, and every other valid size).
void check_order(Report& rep) {
  const int heads[] = {1, 7, 8, 12, 16, 24, 32, 64, 96, 128, 256};
  const int tiles[] = {1, 2, 3, 5, 8, 16, 17, 32, 64, 128};
  const int residents[] = {8, 16, 32, 64, 96};
  int cases = 0;
  for (int BH : heads)
    for (int nq : tiles)
      for (int res : residents) {
        const int pick = head_group_size(res, BH, nq);
        if ((pick == 0) != (BH % 8 != 0)) rep.fail("order BH=%d nq=%d res=%d: group size %d", BH, nq, res, pick);
        if (pick > 1 && pick * nq > res) rep.fail("order BH=%d nq=%d res=%d: group of %d exceeds the XCD", BH, nq, res, pick);
        for (int hg = 0; hg <= 32; hg = hg == 0 ? 1 : 2 * hg) {
          if (hg > 0 && BH % (8 * hg) != 0) continue;
          ++cases;
          std::vector<int> seen((size_t)BH * nq, 0);
          std::vector<int> last_qt(8 * 512, 1 << 30);   // per (XCD, group < 512): previous tile
          for (int bid = 0; bid < BH * nq; ++bid) {
            int bh = -1, qt = -1;
            xcd_head_groups(bid, BH, nq, hg, bh, qt);
            if (bh < 0 || bh >= BH || qt < 0 || qt >= nq) {
              rep.fail("order BH=%d nq=%d hg=%d: workgroup %d -> head %d tile %d out of range", BH, nq, hg, bid, bh, qt);
              break;
            }
            ++seen[(size_t)bh * nq + qt];
            if (hg > 0) {
              if (bh % 8 != bid % 8) rep.fail("order BH=%d nq=%d hg=%d: head %d off its XCD", BH, nq, hg, bh);
              const int grp = (bid / 8) / (hg * nq);
              int& prev = last_qt[(size_t)(bid % 8) * 512 + grp];
              if (qt > prev) rep.fail("order BH=%d nq=%d hg=%d: group %d not heaviest first", BH, nq, hg, grp);
              prev = qt;
            }
          }
          for (size_t i = 0; i < seen.size(); ++i)
            if (seen[i] != 1) {
              rep.fail("order BH=%d nq=%d hg=%d: (head, tile) %zu visited %d times", BH, nq, hg, i, seen[i]);
              break;
            }
        }
      }
  rep.note("order: %d (heads, tiles, group size) cases; B4 H32 N4096 at 32 resident workgroups per XCD: group of %d", cases,
           head_group_size(32, 128, 16));

  // Persistent lists: every item of an XCD's list taken by exactly one of
  // its W workgroups; with the causal cost model (steps of 96 keys plus a
  // fixed two per item) the busiest workgroup's total is reported.
  int pcases = 0;
  for (int n_items : {1, 3, 7, 8, 31, 32, 33, 64, 100, 256, 1000})
    for (int W : {1, 2, 5, 8, 32, 64}) {
      ++pcases;
      std::vector<int> taken(n_items, 0);
      for (int j = 0; j < W; ++j)
        for (int r = 0;; ++r) {
          const int k = persistent_item(j, r, W, n_items);
          if (k < 0) {
            if (r * W < n_items && persistent_item(j, r + 1, W, n_items) >= 0)
              rep.fail("persistent n=%d W=%d: workgroup %d stops at round %d before the list ends", n_items, W, j, r);
            break;
          }
          taken[k]++;
        }
      for (int k = 0; k < n_items; ++k)
        if (taken[k] != 1) {
          rep.fail("persistent n=%d W=%d: item %d taken %d times", n_items, W, k, taken[k]);
          break;
        }
    }
  {
    const int num_qt = 16, hg = head_group_size(32, 128, num_qt), W = 32, n = 16 * num_qt;
    double worst = 0, total = 0;
    for (int j = 0; j < W; ++j) {
      double c = 0;
      for (int r = 0;; ++r) {
        const int k = persistent_item(j, r, W, n);
        if (k < 0) break;
        int bh, qt;
        xcd_item(0, k, num_qt, hg, bh, qt);
        c += (double)(((qt + 1) * 256 + 95) / 96) + 2.0;
      }
      worst = c > worst ? c : worst;
      total += c;
    }
    rep.note("persistent: %d list cases; B4 H32 N4096 causal, 32 workgroups per XCD: busiest %.0f of mean %.1f steps", pcases,
             worst, total / W);
  }
}

// The dQ kernel's Q/dO slots: apart from each other and from each group's
// first two block buffers (copied while the slots are read), slots 0-3
// exactly covering the third buffers of both groups (round 0 reads them as
// finite operands of a product with zero dS), all within 8 S bytes.
template <int D>
void check_dq_slots(Report& rep) {
  const int S = 128 * D, slot = 64 * D;
  std::vector<int> cover(8 * S / 16, 0);
  for (int w = 0; w < 8; ++w) {
    const int a = bwd_dq_qslot<D>(w);
    if (a < 0 || a + slot > 8 * S || a % 1024 != 0)
      rep.fail("dq slots D=%d: slot %d at %d outside or misaligned", D, w, a);
    for (int g = 0; g < 2; ++g)
      for (int b = 0; b < 2; ++b) {
        const int lo = g * 3 * S + b * S;
        if (a < lo + S && lo < a + slot) rep.fail("dq slots D=%d: slot %d overlaps group %d buffer %d", D, w, g, b);
      }
    for (int x = a / 16; x < (a + slot) / 16 && x < (int)cover.size(); ++x) cover[x]++;
  }
  for (size_t x = 0; x < cover.size(); ++x)
    if (cover[x] > 1) {
      rep.fail("dq slots D=%d: byte %zu in two slots", D, 16 * x);
      break;
    }
  for (int g = 0; g < 2; ++g)
    for (int x = (g * 3 * S + 2 * S) / 16; x < (g * 3 * S + 3 * S) / 16; ++x)
      if (cover[x] != 1) {
        rep.fail("dq slots D=%d: group %d buffer 2 byte %d not covered by a slot", D, g, 16 * x);
        break;
      }
  rep.note("dq slots D=%d: 8 slots of %d B, third buffers covered, LDS %d B before the block list", D, slot, 8 * S);
}

}  // namespace

extern "C" int fa_layout_check(char* out, int out_len) {
  Report rep;
  // Launched tile widths, and the wider ones that were tried and set aside
  // (d = 64 with 96 and 128 keys, FP8 with 128 keys).
  check_fwd<64, 32>(rep, true);
  check_fwd<64, 64>(rep, true);
  check_fwd<64, 96>(rep, false);
  check_fwd<64, 128>(rep, false);
  check_fwd<128, 32>(rep, true);
  check_fwd<128, 64>(rep, true);
  check_fwd<128, 96>(rep, true);
  check_fwd<128, 128>(rep, false);
  check_fp8<64, 64>(rep, true);
  check_fp8<64, 128>(rep, false);
  check_fp8<128, 64>(rep, true);
  check_fp8<128, 128>(rep, false);
  check_bwd<64>(rep, 32);
  check_bwd<64>(rep, 128);
  check_bwd<128>(rep, 32);
  check_bwd<128>(rep, 128);
  check_bwd_lds<64>(rep);
  check_bwd_lds<128>(rep);
  check_ostage<32>(rep);
  check_ostage<64>(rep);
  check_ostage<128>(rep);
  check_dq_slots<64>(rep);
  check_dq_slots<128>(rep);
  check_order(rep);
  if (out && out_len > 0) {
    strncpy(out, rep.text.c_str(), (size_t)out_len - 1);
    out[out_len - 1] = 0;
  }
  return rep.violations;
}
