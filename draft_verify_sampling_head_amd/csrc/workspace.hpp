// workspace.hpp -- layout of the caller-provided workspace (host and device).
//
// One workspace serves every entry point of a round; the regions below are
// carved at 256-byte boundaries.  All sizes follow the round's capacity
// (R requests, gamma positions, V vocabulary), never the data-dependent
// counts, so nothing has to visit the host.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace dspark {

struct WsLayout {
  size_t header;       // uint32 words: [0] status flags, [1] residual count
  size_t draft_l;      // float2 [R][nch]   chunk (max, scaled sum) / residual masses
  size_t draft_i;      // int32  [R][nch]   chunk argmax (greedy)
  size_t ver_l;        // float2 [R*(gamma+1)][nch]  target-row chunk (max, scaled sum)
  size_t ver_i;        // int32  [R*(gamma+1)][nch]  target-row chunk argmax (greedy)
  size_t lse_t;        // float2 [R*(gamma+1)]       target-row (max, log-normaliser above it)
  size_t rej;          // int32  [R][4]   residual work list: request, position, row, pad
  size_t bar;          // uint32 [1024] grid-barrier flags of the persistent draft, one per workgroup
  size_t total;
};

inline size_t ws_align(size_t x) { return (x + 255) & ~(size_t)255; }

inline WsLayout ws_layout(int R, int gamma, int V) {
  const size_t nch = ((size_t)V + 127) / 128;
  const size_t rows_v = (size_t)R * (size_t)(gamma + 1);
  WsLayout L;
  size_t off = 0;
  L.header = off;  off += ws_align(256);
  L.draft_l = off; off += ws_align((size_t)R * nch * 8);
  L.draft_i = off; off += ws_align((size_t)R * nch * 4);
  L.ver_l = off;   off += ws_align(rows_v * nch * 8);
  L.ver_i = off;   off += ws_align(rows_v * nch * 4);
  L.lse_t = off;   off += ws_align(rows_v * 8);
  L.rej = off;     off += ws_align((size_t)R * 16);
  L.bar = off;     off += ws_align(4 * 1024);
  L.total = off;
  return L;
}

// RNN draft head: the shared layout, then the h part of the cell's projection
// and the recurrent states (used when the caller passes no state buffer).
struct RnnWsLayout {
  size_t P;            // float [R*gamma][3 rank]
  size_t state;        // float [R][gamma][rank]
  size_t total;
};

inline RnnWsLayout rnn_ws_layout(int R, int gamma, int V, int rank) {
  const size_t pos = (size_t)R * (size_t)gamma;
  RnnWsLayout L;
  size_t off = ws_layout(R, gamma, V).total;
  L.P = off;     off += ws_align(pos * 3 * (size_t)rank * 4);
  L.state = off; off += ws_align(pos * (size_t)rank * 4);
  L.total = off;
  return L;
}

}  // namespace dspark
