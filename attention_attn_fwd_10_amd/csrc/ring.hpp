// The schedule of the two-stage K and V rings in LDS of the 16-bit forward
// (head dims up to 128), as tables that the kernel executes and that a
// compile-time checker proves free of stage hazards.
//
// A tile is copied into LDS by every wave of the workgroup (each wave one
// share of the rows, by asynchronous global -> LDS copies) and read by every
// wave.  Waves run unsynchronised between two barriers, so within one barrier
// interval a stage may be written or read, never both: a read beside a write
// could see the stage half old and half new (one wave still reading while
// another's copy lands, or a copy not landed yet when another wave reads).  A
// read must also see the tile it expects, written before the interval and
// completed by a wait for outstanding copies in every wave before the barrier
// that opened the interval.
//
// Tile t (counted from the work item's first tile j0) lives in stage t % 2.
// The tiles [0, n_pipe) need no mask and run software-pipelined; the tiles
// [n_pipe, n_total) run one at a time (with masks), n_pipe <= n_total.
//   prologue:      copy K0, V0 and K1, wait, barrier, scores of tile 0,
//                  barrier (step 0 refills K0's stage with K2);
//   step j:        copy K(j+2) (if j + 2 <= n_pipe and j + 2 < n_total) and
//                  V(j+1), then the scores of tile j+1 (K(j+1)) with the
//                  softmax and P V of tile j (V(j)), wait, barrier
//                  (j + 1 < n_pipe); in the spread form the two copies are
//                  issued by the step's math, between its first score
//                  products, in the same barrier interval;
//   last:          copy V(j+1) (if j + 1 < n_total), softmax and P V of tile
//                  j = n_pipe - 1, wait, barrier;
//   one at a time: (tile n_pipe = 0: copy K0 and V0, wait, barrier) then per
//                  tile j: copy tile j+1 (if j + 1 < n_total), scores,
//                  softmax and P V of tile j, wait, barrier.
#pragma once

namespace attn {
namespace ring {

enum Kind : int {
  kCopyK,     // copy K(j + d) into its stage
  kCopyV,     // copy V(j + d) into its stage
  kCopyKV,    // copy K(j + d) and V(j + d) into their stages
  kScores,    // read K(j + d)
  kStepMath,  // read K(j + d + 1) and V(j + d)
  kLastMath,  // read V(j + d)
  kTileMath,  // read K(j + d) and V(j + d)
  kWait,      // wait for this wave's outstanding copies
  kSync       // workgroup barrier
};
enum Guard : int {
  kAlways,
  kLtTotal,      // tile j + d < n_total
  kLePipeLtTotal  // tile j + d <= n_pipe and < n_total
};
// in_math: a copy that the math op of the same table issues itself (spread
// between its instructions) instead of one issued before it.  It lies in the
// same barrier interval either way, so the hazard rules below treat it alike.
struct Op {
  int kind, d, guard;
  int in_math = 0;
};

constexpr Op kPrologue[] = {{kCopyK, 0, kAlways}, {kCopyV, 0, kAlways}, {kCopyK, 1, kLtTotal}, {kWait, 0, kAlways},
                            {kSync, 0, kAlways},  {kScores, 0, kAlways}, {kSync, 0, kAlways}};
constexpr Op kStep[] = {{kCopyK, 2, kLePipeLtTotal}, {kCopyV, 1, kAlways}, {kStepMath, 0, kAlways},
                        {kWait, 0, kAlways},        {kSync, 0, kAlways}};
constexpr Op kStepSpread[] = {{kCopyK, 2, kLePipeLtTotal, 1}, {kCopyV, 1, kAlways, 1}, {kStepMath, 0, kAlways},
                              {kWait, 0, kAlways},           {kSync, 0, kAlways}};
constexpr Op kLast[] = {{kCopyV, 1, kLtTotal}, {kLastMath, 0, kAlways}, {kWait, 0, kAlways}, {kSync, 0, kAlways}};
constexpr Op kTileStart[] = {{kCopyKV, 0, kAlways}, {kWait, 0, kAlways}, {kSync, 0, kAlways}};
constexpr Op kTile[] = {{kCopyKV, 1, kLtTotal}, {kTileMath, 0, kAlways}, {kWait, 0, kAlways}, {kSync, 0, kAlways}};

// a table as a type, so that its ops are constant expressions where it is run
template <const auto& T>
struct Table {
  static constexpr int size = sizeof(T) / sizeof(T[0]);
  static constexpr Op at(int i) { return T[i]; }
  // position of op i among the table's in_math copies, and their number
  static constexpr int in_math_index(int i) {
    int n = 0;
    for (int k = 0; k < i; ++k) n += T[k].in_math;
    return n;
  }
  static constexpr int in_math_count = in_math_index(size);
};

constexpr bool guard_ok(int guard, int tile, int n_pipe, int n_total) {
  return guard == kAlways ? true : guard == kLtTotal ? tile < n_total : tile <= n_pipe && tile < n_total;
}

// ---- compile-time hazard check ------------------------------------------------
// Per stage (K0, K1, V0, V1): the tile last written, whether every wave has
// waited for that copy, whether a barrier has followed that wait, and whether
// the stage was written or read in the current barrier interval.
struct Stage {
  int tile = -1;
  bool landed = false, visible = false, written = false, read = false;
};
struct Sim {
  Stage st[4];  // K0, K1, V0, V1
  bool ok = true;
  constexpr void write(int s, int tile) {
    if (st[s].read || st[s].written) ok = false;  // another wave may still read it
    st[s].tile = tile;
    st[s].landed = st[s].visible = false;
    st[s].written = true;
  }
  constexpr void read(int s, int tile) {
    if (st[s].written || !st[s].visible || st[s].tile != tile) ok = false;
    st[s].read = true;
  }
  constexpr void wait() {
    for (Stage& x : st)
      if (x.tile >= 0) x.landed = true;
  }
  constexpr void sync() {
    for (Stage& x : st) {
      x.visible = x.landed;
      x.written = x.read = false;
    }
  }
  template <int N>
  constexpr void run(const Op (&ops)[N], int j, int n_pipe, int n_total) {
    for (int i = 0; i < N; ++i) {
      const Op& o = ops[i];
      const int t = j + o.d;
      if (!guard_ok(o.guard, t, n_pipe, n_total)) continue;
      switch (o.kind) {
        case kCopyK: write(t % 2, t); break;
        case kCopyV: write(2 + t % 2, t); break;
        case kCopyKV:
          write(t % 2, t);
          write(2 + t % 2, t);
          break;
        case kScores: read(t % 2, t); break;
        case kStepMath:
          read((t + 1) % 2, t + 1);
          read(2 + t % 2, t);
          break;
        case kLastMath: read(2 + t % 2, t); break;
        case kTileMath:
          read(t % 2, t);
          read(2 + t % 2, t);
          break;
        case kWait: wait(); break;
        default: sync(); break;
      }
    }
  }
};

// The whole key loop of one work item with n_total tiles, the first n_pipe
// of them pipelined, run through the given tables.
template <int A, int B, int C, int D, int E>
constexpr bool schedule_ok(int n_pipe, int n_total, const Op (&pro)[A], const Op (&step)[B], const Op (&last)[C],
                           const Op (&start)[D], const Op (&tile)[E]) {
  Sim s;
  if (n_pipe > 0) {
    s.run(pro, 0, n_pipe, n_total);
    for (int j = 0; j + 1 < n_pipe; ++j) s.run(step, j, n_pipe, n_total);
    s.run(last, n_pipe - 1, n_pipe, n_total);
  } else {
    s.run(start, 0, n_pipe, n_total);
  }
  for (int j = n_pipe; j < n_total; ++j) s.run(tile, j, n_pipe, n_total);
  return s.ok;
}

template <int A, int B, int C, int D, int E>
constexpr bool schedule_ok_all(const Op (&pro)[A], const Op (&step)[B], const Op (&last)[C], const Op (&start)[D],
                               const Op (&tile)[E]) {
  for (int n_total = 1; n_total <= 9; ++n_total)
    for (int n_pipe = 0; n_pipe <= n_total; ++n_pipe)
      if (!schedule_ok(n_pipe, n_total, pro, step, last, start, tile)) return false;
  return true;
}

static_assert(schedule_ok_all(kPrologue, kStep, kLast, kTileStart, kTile),
              "the K/V ring schedule reads a stage beside a write to it, or before its copy is complete");
static_assert(schedule_ok_all(kPrologue, kStepSpread, kLast, kTileStart, kTile),
              "the spread K/V ring schedule reads a stage beside a write to it, or before its copy is complete");

}  // namespace ring
}  // namespace attn
