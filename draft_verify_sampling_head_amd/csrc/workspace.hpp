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
  size_t header;       // uint32 words: [0] status flags, [1] residual count,
                       // [2] pipelined-draft epoch, [3] verify epoch, [4] epoch
                       // of the last verify whose rows all finished, [5] verify
                       // rows finished
  size_t draft_l;      // float2 [R][nch]   chunk (max, scaled sum) / residual masses
  size_t draft_i;      // int32  [R][nch]   chunk argmax (greedy)
  size_t ver_l;        // float2 [R*(gamma+1)][nch]  target-row chunk (max, scaled sum)
  size_t ver_i;        // int32  [R*(gamma+1)][nch]  target-row chunk argmax (greedy)
  size_t lse_t;        // float2 [R*(gamma+1)]       target-row (max, log-normaliser above it)
  size_t rej;          // int32  [R][4]   residual work list: request, position, row, pad
  size_t vaux;         // int32  [R][2 + gamma] verify: rows finished and bonus token per
                       // request, outcome of every tested position
  size_t bar;          // uint32 [1024] grid-barrier flags of the persistent draft, one per workgroup
  size_t rec;          // 16-byte [2][R][ceil(V/512)] per-slice records of the pipelined draft
  size_t total;
};

// Number of 512-entry vocabulary slices (one per workgroup of the persistent draft).
inline size_t ws_nslice(int V) { return ((size_t)V + 511) / 512; }

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
  L.vaux = off;    off += ws_align((size_t)R * (gamma + 2) * 4);
  L.bar = off;     off += ws_align(4 * 1024);
  L.rec = off;     off += ws_align(2 * (size_t)R * ws_nslice(V) * 16);
  L.total = off;
  return L;
}

// The regions the draft uses, as pointers.  rows_l / rows_i (statistics of
// all R gamma rows at rank 0, one launch) may be null: the rank-0 draft then
// runs one statistics launch per position in draft_l / draft_i.
struct DraftWs {
  uint32_t* status;    // status word
  void* draft_l;       // float2 [R][nch]
  void* draft_i;       // int32  [R][nch]
  uint32_t* bar;       // uint32 [1024] grid-barrier flags
  void* rec;           // 16-byte [2][R][ceil(V/512)]
  void* rows_l;        // nullable float2 [R*gamma][nch]
  void* rows_i;        // nullable int32  [R*gamma][nch]
};

inline DraftWs draft_ws(void* ws, int R, int gamma, int V) {
  const WsLayout L = ws_layout(R, gamma, V);
  char* w = reinterpret_cast<char*>(ws);
  DraftWs d;
  d.status = reinterpret_cast<uint32_t*>(w + L.header);
  d.draft_l = w + L.draft_l;
  d.draft_i = w + L.draft_i;
  d.bar = reinterpret_cast<uint32_t*>(w + L.bar);
  d.rec = w + L.rec;
  d.rows_l = w + L.ver_l;      // the target-row statistics, unused until the verify
  d.rows_i = w + L.ver_i;
  return d;
}

// The draft alone in a compact layout (no rank-0 all-rows region):
// header, draft_l, draft_i, barrier flags, records.  Returns the bytes needed.
inline size_t draft_ws_compact(char* base, int R, int V, DraftWs* d) {
  const size_t nch = ((size_t)V + 127) / 128;
  size_t off = 0;
  const size_t h = off;  off += ws_align(256);
  const size_t l = off;  off += ws_align((size_t)R * nch * 8);
  const size_t i = off;  off += ws_align((size_t)R * nch * 4);
  const size_t b = off;  off += ws_align(4 * 1024);
  const size_t r = off;  off += ws_align(2 * (size_t)R * ws_nslice(V) * 16);
  if (d) {
    d->status = reinterpret_cast<uint32_t*>(base + h);
    d->draft_l = base + l;
    d->draft_i = base + i;
    d->bar = reinterpret_cast<uint32_t*>(base + b);
    d->rec = base + r;
    d->rows_l = nullptr;
    d->rows_i = nullptr;
  }
  return off;
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
