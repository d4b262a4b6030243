/*
 * dspark_oracle.cpp -- plain CPU oracle for one confidence-scheduled
 * speculative-decoding round (Markov draft head, confidence head, prefix
 * scheduler, rejection-sampling verify, ragged pack).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no source with the HIP library (no headers, helpers,
 * tables or constants); the two sides meet only through their documented
 * definitions and through seeded inputs.
 *
 * Style: single thread, no blocking, no fusion.  Every floating-point input is
 * widened exactly to double and every sum runs in double in ascending index
 * order.  Where a floating-point value decides an integer (an argmax, a Gumbel
 * pick, an accept test) the decision is taken on the float32 rounding of the
 * double value, the precision the GPU kernels decide in; the double gap
 * between the two best candidates is reported as that decision's margin.
 *
 * Sources (the web pages collected on DSpark; cited by page and section):
 *  [P3] papercache.org summary of "DSpark: Confidence-Scheduled Speculative
 *       Decoding with Semi-Autoregressive Generation" (arXiv 2607.05147):
 *       sections "Background" (acceptance rule), "Method details" (causal block
 *       distribution, Markov head, confidence head, STS calibration, hardware-
 *       aware prefix scheduler, Algorithm 1) and Appendix A.
 *  [P1] backyes.github.io "MTP algorithm survey", section 2.2 (rejection
 *       sampling: residual distribution, greedy reduction, bonus token, tau=m+1).
 *  [P2] bevisy.github.io DeepSpec analysis, section 2.2 (markov_rank=0 is the
 *       DFlash case: independent per-position sampling).
 *  [P4] modelscope/CSDN DSpark article, section 3.3 (flatten + marker tensors).
 *
 * Random numbers: the pages do not define a random stream.  This oracle uses
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
 * as 1, 2, 3", SC'11) written from that paper's definition:
 *   key     = (lo32(seed), hi32(seed))
 *   counter = (idx >> 2, k | tag << 16, request, lo32(round)),  word = idx & 3
 *   u       = (word + 1/2) * 2^-32 in (0, 1)
 *   G       = -log(-log(u))                      (standard Gumbel)
 * Sampling from softmax(score) uses the chunked Gumbel-max rule (CGM): with
 * chunks of CHUNK consecutive entries, first pick a chunk by Gumbel-max over
 * the chunk log-masses, then an entry inside it by Gumbel-max over the scores.
 * P(chunk) * P(entry | chunk) is exactly softmax(score) (Gumbel-max theorem
 * applied twice), so CGM is an exact categorical sampler.
 */
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>
#include <algorithm>

namespace {

constexpr int64_t CHUNK = 128;   // chunk width of the chunked Gumbel-max rule

enum Tag : uint32_t {
    TAG_DRAFT_CHUNK = 1, TAG_DRAFT_ELEM = 2, TAG_ACCEPT = 3,
    TAG_RESID_CHUNK = 4, TAG_RESID_ELEM = 5, TAG_BONUS_CHUNK = 6, TAG_BONUS_ELEM = 7
};

const double NEG_INF = -std::numeric_limits<double>::infinity();
const double POS_INF = std::numeric_limits<double>::infinity();

// ---------------------------------------------------------------- Philox ---
// Ten rounds of the Philox 4x32 S-box: two 32x32->64 products, the halves
// cross-xored with the other counter words and the round key; the key is
// bumped by the Weyl constants (golden ratio, sqrt(3)-1) between rounds.
void philox4x32_10(const uint32_t ctr_in[4], uint32_t key0, uint32_t key1, uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = hi1 ^ c1 ^ key0;
        const uint32_t n1 = lo1;
        const uint32_t n2 = hi0 ^ c3 ^ key1;
        const uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        key0 += 0x9E3779B9u;
        key1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

uint32_t stream_word(uint64_t seed, uint64_t round, uint32_t tag, uint32_t req,
                     uint32_t k, uint32_t idx) {
    const uint32_t ctr[4] = {idx >> 2, k | (tag << 16), req, (uint32_t)round};
    uint32_t out[4];
    philox4x32_10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32), out);
    return out[idx & 3u];
}

double uniform01(uint32_t word) { return ((double)word + 0.5) * 0x1p-32; }

double gumbel(uint32_t word) { return -std::log(-std::log(uniform01(word))); }

// ------------------------------------------------------------- helpers ----
double logsumexp(const double* v, int64_t n) {
    double mx = NEG_INF;
    for (int64_t i = 0; i < n; ++i) mx = std::max(mx, v[i]);
    if (mx == NEG_INF) return NEG_INF;
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += std::exp(v[i] - mx);
    return mx + std::log(s);
}

// First index whose float32-rounded value is maximal (ties -> lower index);
// entries equal to -inf are skipped.  *gap = double gap between the best and
// the second-best candidate (+inf if fewer than two).
int64_t argmax_f32_decision(const double* v, int64_t n, double* gap) {
    int64_t best = -1;
    float bestf = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (v[i] == NEG_INF) continue;
        const float f = (float)v[i];
        if (best < 0 || f > bestf) { best = i; bestf = f; }
    }
    if (gap) {
        double a = NEG_INF, b = NEG_INF;
        for (int64_t i = 0; i < n; ++i) {
            if (v[i] > a) { b = a; a = v[i]; } else if (v[i] > b) { b = v[i]; }
        }
        *gap = (b == NEG_INF) ? POS_INF : (a - b);
    }
    return best;
}

// Chunked Gumbel-max sample from softmax(score[0..n)).  Entries equal to -inf
// carry no mass and are never chosen.  Returns -1 only if all entries are -inf.
int64_t cgm_sample(const double* score, int64_t n, uint64_t seed, uint64_t round,
                   uint32_t tag_chunk, uint32_t tag_elem, uint32_t req, uint32_t k,
                   double* margin) {
    const int64_t nch = (n + CHUNK - 1) / CHUNK;
    int64_t cstar = 0;
    double m_chunk = POS_INF;
    if (nch >= 2) {
        std::vector<double> key(nch);
        for (int64_t c = 0; c < nch; ++c) {
            const int64_t lo = c * CHUNK, hi = std::min(n, lo + CHUNK);
            const double L = logsumexp(score + lo, hi - lo);
            key[c] = (L == NEG_INF) ? NEG_INF
                                    : L + gumbel(stream_word(seed, round, tag_chunk, req, k, (uint32_t)c));
        }
        cstar = argmax_f32_decision(key.data(), nch, &m_chunk);
        if (cstar < 0) { if (margin) *margin = POS_INF; return -1; }
    }
    const int64_t lo = cstar * CHUNK, hi = std::min(n, lo + CHUNK);
    std::vector<double> key(hi - lo);
    for (int64_t v = lo; v < hi; ++v)
        key[v - lo] = (score[v] == NEG_INF) ? NEG_INF
                      : score[v] + gumbel(stream_word(seed, round, tag_elem, req, k, (uint32_t)v));
    double m_elem = POS_INF;
    const int64_t j = argmax_f32_decision(key.data(), hi - lo, &m_elem);
    if (margin) *margin = std::min(m_chunk, m_elem);
    return j < 0 ? -1 : lo + j;
}

// Base logits plus Markov transition bias for one block position:
//   out[v] = U_k[v] + sum_i W1[prev][i] * W2[i][v]        ([P3] Method details,
// causal block distribution and Markov head: B(x_{k-1}, .) = W1[x_{k-1}] W2).
// W2 is passed transposed, W2t[v][i] = W2[i][v] (the [V][r] layout of a linear
// layer r -> V).  rank == 0 means no head (the DFlash case, [P2] 2.2).
void markov_scores(int64_t V, int rank, const float* Uk, const float* W1, const float* W2t,
                   int32_t prev, double* out) {
    const float* e = (rank > 0) ? W1 + (int64_t)prev * rank : nullptr;
    for (int64_t v = 0; v < V; ++v) {
        double b = 0.0;
        if (rank > 0) {
            const float* w = W2t + v * rank;
            for (int i = 0; i < rank; ++i) b += (double)e[i] * (double)w[i];
        }
        out[v] = (double)Uk[v] + b;
    }
}

// Residual weights at a rejected position ([P1] 2.2: q = norm(max(0, p_t - p_d))).
// lt = target logits / T with normalizer lse_t; s = tempered draft scores with
// the draft's normalizer lse_d.  Returns the total unnormalised mass.
double residual_weights(int64_t V, const double* lt, double lse_t, const double* s,
                        double lse_d, double* q) {
    double tot = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        const double d = std::exp(lt[v] - lse_t) - std::exp(s[v] - lse_d);
        q[v] = d > 0.0 ? d : 0.0;
        tot += q[v];
    }
    return tot;
}

}  // namespace

extern "C" {

// ------------------------------------------------------- random stream ----
void orc_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
    philox4x32_10(ctr, key[0], key[1], out);
}

uint32_t orc_stream_word(uint64_t seed, uint64_t round, uint32_t tag, uint32_t req,
                         uint32_t k, uint32_t idx) {
    return stream_word(seed, round, tag, req, k, idx);
}

double orc_gumbel(uint64_t seed, uint64_t round, uint32_t tag, uint32_t req, uint32_t k,
                  uint32_t idx) {
    return gumbel(stream_word(seed, round, tag, req, k, idx));
}

int64_t orc_chunk_width(void) { return CHUNK; }

// CGM sample from softmax(score); tag_chunk/tag_elem select the stream.
int64_t orc_cgm(const double* score, int64_t n, uint64_t seed, uint64_t round,
                uint32_t tag_chunk, uint32_t tag_elem, uint32_t req, uint32_t k,
                double* margin) {
    return cgm_sample(score, n, seed, round, tag_chunk, tag_elem, req, k, margin);
}

// The same CGM draw for request ids req0 .. req0+count-1 (independent streams);
// used to gather sampling statistics in one call.
void orc_cgm_batch(const double* score, int64_t n, uint64_t seed, uint64_t round,
                   uint32_t tag_chunk, uint32_t tag_elem, uint32_t req0, int64_t count,
                   uint32_t k, int64_t* out) {
    for (int64_t q = 0; q < count; ++q)
        out[q] = cgm_sample(score, n, seed, round, tag_chunk, tag_elem, req0 + (uint32_t)q, k,
                            nullptr);
}

// ------------------------------------------------------ distributions -----
// Draft distribution of one block position ([P3] Method details, causal block
// distribution): p(v) = softmax((U_k + W1[prev] W2) / T)(v), T > 0.
void orc_draft_row(int64_t V, int rank, double T, const float* Uk, const float* W1,
                   const float* W2t, int32_t prev, double* p_out) {
    std::vector<double> s(V);
    markov_scores(V, rank, Uk, W1, W2t, prev, s.data());
    for (int64_t v = 0; v < V; ++v) s[v] /= T;
    const double lse = logsumexp(s.data(), V);
    for (int64_t v = 0; v < V; ++v) p_out[v] = std::exp(s[v] - lse);
}

// Normalised residual distribution for target logits t (divided by T inside)
// and draft scores s (tempered, normaliser lse_d).  Zero residual mass falls
// back to the target distribution.  Returns the unnormalised mass.
double orc_residual_row(int64_t V, double T, const float* t, const double* s, double lse_d,
                        double* q_out) {
    std::vector<double> lt(V);
    for (int64_t v = 0; v < V; ++v) lt[v] = (double)t[v] / T;
    const double lse_t = logsumexp(lt.data(), V);
    const double tot = residual_weights(V, lt.data(), lse_t, s, lse_d, q_out);
    if (tot > 0.0) {
        for (int64_t v = 0; v < V; ++v) q_out[v] /= tot;
    } else {
        for (int64_t v = 0; v < V; ++v) q_out[v] = std::exp(lt[v] - lse_t);
    }
    return tot;
}

// ---------------------------------------------------------------- draft ---
// Markov draft head over a block ([P3] Method details: causal block
// distribution and Markov head; anchor x_0 is the last round's bonus token).
//  U      [R][gamma][V]  base logits U_1..U_gamma
//  W1     [V][rank]      embedding table, W2t [V][rank] (= W2 transposed)
//  x0     [R]            anchors
//  req_ids[R] nullable   request index used in the random stream (default i)
//  force_x[R][gamma+1]   nullable; entries >= 0 replace the sample (lock-step)
// Out: x [R][gamma+1] (x[i][0] = anchor), logp_d, lse_d, margin [R][gamma];
//      x_own [R][gamma+1] nullable: the oracle's own choice at each position
//      given the (possibly forced) prefix.
// T > 0: x_k ~ softmax(s), s = (U_k + bias) / T, logp_d = s(x_k) - lse_d.
// T == 0: x_k = first argmax of U_k + bias; logp_d = 0; lse_d = max score.
int orc_draft_markov(int R, int gamma, int64_t V, int rank, double T, uint64_t seed,
                     uint64_t round, const float* U, const float* W1, const float* W2t,
                     const int32_t* x0, const int32_t* req_ids, const int32_t* force_x,
                     int32_t* x, double* logp_d, double* lse_d, double* margin, int32_t* x_own) {
    if (R < 0 || gamma < 1 || V < 1 || rank < 0 || !(T >= 0.0)) return 1;
    std::vector<double> s(V);
    for (int i = 0; i < R; ++i) {
        const uint32_t rid = req_ids ? (uint32_t)req_ids[i] : (uint32_t)i;
        int32_t prev = x0[i];
        x[(int64_t)i * (gamma + 1)] = prev;
        if (x_own) x_own[(int64_t)i * (gamma + 1)] = prev;
        for (int k = 1; k <= gamma; ++k) {
            const float* Uk = U + ((int64_t)i * gamma + (k - 1)) * V;
            markov_scores(V, rank, Uk, W1, W2t, prev, s.data());
            int64_t xk;
            double lp, lse, mg;
            if (T > 0.0) {
                for (int64_t v = 0; v < V; ++v) s[v] /= T;
                lse = logsumexp(s.data(), V);
                xk = cgm_sample(s.data(), V, seed, round, TAG_DRAFT_CHUNK, TAG_DRAFT_ELEM,
                                rid, (uint32_t)k, &mg);
                if (x_own) x_own[(int64_t)i * (gamma + 1) + k] = (int32_t)xk;
                if (force_x && force_x[(int64_t)i * (gamma + 1) + k] >= 0)
                    xk = force_x[(int64_t)i * (gamma + 1) + k];
                lp = s[xk] - lse;
            } else {
                xk = argmax_f32_decision(s.data(), V, &mg);
                if (x_own) x_own[(int64_t)i * (gamma + 1) + k] = (int32_t)xk;
                if (force_x && force_x[(int64_t)i * (gamma + 1) + k] >= 0)
                    xk = force_x[(int64_t)i * (gamma + 1) + k];
                double mx = NEG_INF;
                for (int64_t v = 0; v < V; ++v) mx = std::max(mx, s[v]);
                lp = 0.0;
                lse = mx;
            }
            x[(int64_t)i * (gamma + 1) + k] = (int32_t)xk;
            const int64_t o = (int64_t)i * gamma + (k - 1);
            if (logp_d) logp_d[o] = lp;
            if (lse_d) lse_d[o] = lse;
            if (margin) margin[o] = mg;
            prev = (int32_t)xk;
        }
    }
    return 0;
}

// -------------------------------------------------------------- RNN head ---
// RNN draft head ([P3] Method details, RNN head): a recurrent state carries
// the whole in-block prefix.  With z_k = [s_{k-1} ; W1[x_{k-1}] ; h_k] (length
// 2r + d, s_0 = 0) and one projection Wr [3r][2r + d] whose rows are the gate,
// candidate and output parts (no bias terms),
//   g = sigmoid(Wr_g z_k),  s_k = g * s_{k-1} + (1 - g) * tanh(Wr_c z_k),
//   e_k = tanh(Wr_o z_k),   bias_k(v) = sum_j e_k[j] W2t[v][j]  (= W2^T e_k),
// then x_k is sampled from softmax((U_k + bias_k) / T) as for the Markov head
// (same random stream).  Reading: e_k is the activation handed to the W2
// projection in the model's dtype; with bf16_e it is rounded to bf16 (round to
// nearest even), and e_margin reports, per element, the absolute distance of
// the unrounded value to the nearest bf16 rounding boundary (the same absolute
// scale as the other decision margins: an error in the pre-activation moves e
// by an absolute amount whatever its size)
// (+inf when not rounded).  force_e (nullable, [R][gamma][r]) replaces e_k
// after rounding (lock-step checking); force_x as for the Markov head.
// Out: x, logp_d, lse_d, margin, x_own as orc_draft_markov; e [R][gamma][r]
//      (the features used), s [R][gamma][r] (states s_1..s_gamma), e_margin.
static double bf16_round(double v, double* abs_margin) {
    // round to bf16 (8 significant bits) with ties to even, from the exact value
    if (v == 0.0 || !std::isfinite(v)) { if (abs_margin) *abs_margin = POS_INF; return v; }
    int ex;
    const double m = std::frexp(std::fabs(v), &ex);     // |v| = m 2^ex, m in [0.5, 1)
    const double scaled = m * 256.0;                     // 8 bits: [128, 256)
    const double fl = std::floor(scaled);
    const double frac = scaled - fl;
    double r = fl;
    if (frac > 0.5 || (frac == 0.5 && std::fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
    if (abs_margin) *abs_margin = std::ldexp(std::fabs(frac - 0.5), ex - 8);   // in units of v
    return std::copysign(std::ldexp(r / 256.0, ex), v);
}

int orc_draft_rnn(int R, int gamma, int64_t V, int rank, int d, double T, uint64_t seed,
                  uint64_t round, const float* U, const float* W1, const float* W2t,
                  const float* Wr, const float* h, const int32_t* x0, const int32_t* req_ids,
                  const int32_t* force_x, const float* force_e, int bf16_e, int32_t* x,
                  double* logp_d, double* lse_d, double* margin, int32_t* x_own, double* e_out,
                  double* s_out, double* e_margin) {
    if (R < 0 || gamma < 1 || V < 1 || rank < 1 || d < 1 || !(T >= 0.0)) return 1;
    const int nz = 2 * rank + d;
    std::vector<double> sc(V), z(nz), st(rank), e(rank);
    for (int i = 0; i < R; ++i) {
        const uint32_t rid = req_ids ? (uint32_t)req_ids[i] : (uint32_t)i;
        int32_t prev = x0[i];
        x[(int64_t)i * (gamma + 1)] = prev;
        if (x_own) x_own[(int64_t)i * (gamma + 1)] = prev;
        std::fill(st.begin(), st.end(), 0.0);
        for (int k = 1; k <= gamma; ++k) {
            const int64_t o = (int64_t)i * gamma + (k - 1);
            for (int j = 0; j < rank; ++j) z[j] = st[j];
            for (int j = 0; j < rank; ++j) z[rank + j] = (double)W1[(int64_t)prev * rank + j];
            for (int j = 0; j < d; ++j) z[2 * rank + j] = (double)h[o * d + j];
            std::vector<double> gs(rank);
            for (int j = 0; j < rank; ++j) {
                double pg = 0.0, pc = 0.0, po = 0.0;
                const float* rg = Wr + (int64_t)j * nz;
                const float* rc = Wr + (int64_t)(rank + j) * nz;
                const float* ro = Wr + (int64_t)(2 * rank + j) * nz;
                for (int q = 0; q < nz; ++q) {
                    pg += (double)rg[q] * z[q];
                    pc += (double)rc[q] * z[q];
                    po += (double)ro[q] * z[q];
                }
                const double g = 1.0 / (1.0 + std::exp(-pg));
                gs[j] = g * st[j] + (1.0 - g) * std::tanh(pc);
                double mgn = POS_INF;
                double ev = std::tanh(po);
                if (bf16_e) ev = bf16_round(ev, &mgn);
                if (force_e) ev = (double)force_e[o * rank + j];
                e[j] = ev;
                if (e_margin) e_margin[o * rank + j] = mgn;
            }
            st = gs;
            for (int j = 0; j < rank; ++j) {
                if (e_out) e_out[o * rank + j] = e[j];
                if (s_out) s_out[o * rank + j] = st[j];
            }
            const float* Uk = U + o * V;
            for (int64_t v = 0; v < V; ++v) {
                double b = 0.0;
                const float* w = W2t + v * rank;
                for (int j = 0; j < rank; ++j) b += e[j] * (double)w[j];
                sc[v] = (double)Uk[v] + b;
            }
            int64_t xk;
            double lp, lse, mg;
            if (T > 0.0) {
                for (int64_t v = 0; v < V; ++v) sc[v] /= T;
                lse = logsumexp(sc.data(), V);
                xk = cgm_sample(sc.data(), V, seed, round, TAG_DRAFT_CHUNK, TAG_DRAFT_ELEM, rid,
                                (uint32_t)k, &mg);
                if (x_own) x_own[(int64_t)i * (gamma + 1) + k] = (int32_t)xk;
                if (force_x && force_x[(int64_t)i * (gamma + 1) + k] >= 0)
                    xk = force_x[(int64_t)i * (gamma + 1) + k];
                lp = sc[xk] - lse;
            } else {
                xk = argmax_f32_decision(sc.data(), V, &mg);
                if (x_own) x_own[(int64_t)i * (gamma + 1) + k] = (int32_t)xk;
                if (force_x && force_x[(int64_t)i * (gamma + 1) + k] >= 0)
                    xk = force_x[(int64_t)i * (gamma + 1) + k];
                double mx = NEG_INF;
                for (int64_t v = 0; v < V; ++v) mx = std::max(mx, sc[v]);
                lp = 0.0;
                lse = mx;
            }
            x[(int64_t)i * (gamma + 1) + k] = (int32_t)xk;
            if (logp_d) logp_d[o] = lp;
            if (lse_d) lse_d[o] = lse;
            if (margin) margin[o] = mg;
            prev = (int32_t)xk;
        }
    }
    return 0;
}

// ----------------------------------------------------------- confidence ---
// c_k = sigmoid(w^T [h_k ; W1[x_{k-1}]] / t_k)  ([P3] Method details, confidence
// head; optional per-position STS temperatures t_k, default 1).  The result is
// rounded to float32 (the scheduler consumes float32 confidences).
void orc_confidence(int R, int gamma, int d, int rank, const float* h, const float* W1,
                    const float* w, const float* sts_T, const int32_t* x, float* c,
                    double* z_out) {
    for (int i = 0; i < R; ++i) {
        for (int k = 1; k <= gamma; ++k) {
            const float* hk = h + ((int64_t)i * gamma + (k - 1)) * d;
            double z = 0.0;
            for (int j = 0; j < d; ++j) z += (double)w[j] * (double)hk[j];
            if (rank > 0) {
                const float* e = W1 + (int64_t)x[(int64_t)i * (gamma + 1) + (k - 1)] * rank;
                for (int j = 0; j < rank; ++j) z += (double)w[d + j] * (double)e[j];
            }
            const double t = sts_T ? (double)sts_T[k - 1] : 1.0;
            const int64_t o = (int64_t)i * gamma + (k - 1);
            c[o] = (float)(1.0 / (1.0 + std::exp(-z / t)));
            if (z_out) z_out[o] = z;
        }
    }
}

// ------------------------------------------------------------ scheduler ---
// Hardware-aware prefix scheduler, [P3] Method details ("greedy solution and
// causality", Algorithm 1):
//   a_{r,j} = prod_{i<=j} c_{r,i}, evaluated left to right in float32;
//   E = {(r,j) : a_{r,j} > 0} sorted by a descending (ties: r, then j ascending);
//   start from B = R, tau = R, Theta_best = R * SPS(R); admit candidates in
//   order, B += 1, tau += a; Theta = tau * SPS(B); on improvement record
//   ell_r = j, otherwise stop (early stop).  B > N_max means capacity exceeded
//   (Theta = 0).  tau is kept in 2^-32 fixed point (an int64), so that the sums
//   are exact and independent of order; Theta is one double product.
// mode 0 = Algorithm 1.  mode 1 = the no-early-stop global search that
// Appendix A uses as a counterexample (best Theta over all sorted prefixes);
// it exists only as a negative control for tests.
// Out: ell [R]; a [R][gamma] (nullable); N = sum(1+ell); Theta_best;
//      margin = smallest relative |Theta - Theta_best| / Theta_best among the
//      comparisons made (nullable).
int orc_prefix_schedule(int R, int gamma, const float* c, const double* sps, int N_max,
                        int enabled, int mode, int32_t* ell, float* a_out, int32_t* N_out,
                        double* theta_best, double* margin) {
    if (R < 0 || gamma < 1 || N_max < R) return 1;
    std::vector<float> a((size_t)R * gamma);
    for (int r = 0; r < R; ++r) {
        float acc = 1.0f;
        for (int j = 1; j <= gamma; ++j) {
            acc = acc * c[(int64_t)r * gamma + (j - 1)];   // float32 product
            a[(size_t)r * gamma + (j - 1)] = acc;
        }
    }
    if (a_out) std::memcpy(a_out, a.data(), a.size() * sizeof(float));
    auto fix = [](float av) -> int64_t { return (int64_t)std::llrint((double)av * 0x1p32); };
    auto theta_of = [&](int64_t tau_fx, int64_t B) -> double {
        if (B > N_max) return 0.0;
        return ((double)tau_fx * 0x1p-32) * sps[B];
    };
    double mg = POS_INF;
    if (!enabled) {
        int64_t tau = (int64_t)R << 32;
        for (size_t q = 0; q < a.size(); ++q) tau += fix(a[q]);
        for (int r = 0; r < R; ++r) ell[r] = gamma;
        if (N_out) *N_out = R * (gamma + 1);
        if (theta_best) *theta_best = theta_of(tau, (int64_t)R * (gamma + 1));
        if (margin) *margin = mg;
        return 0;
    }
    struct Cand { float a; int r; int j; };
    std::vector<Cand> E;
    for (int r = 0; r < R; ++r)
        for (int j = 1; j <= gamma; ++j) {
            const float av = a[(size_t)r * gamma + (j - 1)];
            if (av > 0.0f) E.push_back({av, r, j});
        }
    std::sort(E.begin(), E.end(), [](const Cand& p, const Cand& q) {
        if (p.a != q.a) return p.a > q.a;
        if (p.r != q.r) return p.r < q.r;
        return p.j < q.j;
    });
    for (int r = 0; r < R; ++r) ell[r] = 0;
    int64_t tau = (int64_t)R << 32;
    int64_t B = R;
    double best = theta_of(tau, B);
    if (mode == 0) {
        for (const Cand& e : E) {
            B += 1;
            tau += fix(e.a);
            const double th = theta_of(tau, B);
            if (best > 0.0) mg = std::min(mg, std::fabs(th - best) / best);
            if (th > best) {
                best = th;
                ell[e.r] = e.j;
            } else {
                break;
            }
        }
    } else {
        // global search: keep the best prefix of the whole sorted list
        std::vector<int32_t> cur(R, 0);
        size_t best_n = 0;
        for (size_t n = 0; n < E.size(); ++n) {
            B += 1;
            tau += fix(E[n].a);
            const double th = theta_of(tau, B);
            if (th > best) { best = th; best_n = n + 1; }
        }
        for (size_t n = 0; n < best_n; ++n) ell[E[n].r] = E[n].j;
    }
    int64_t N = 0;
    for (int r = 0; r < R; ++r) N += 1 + ell[r];
    if (N_out) *N_out = (int32_t)N;
    if (theta_best) *theta_best = best;
    if (margin) *margin = mg;
    return 0;
}

// ------------------------------------------------ asynchronous scheduler ---
// The scheduler as deployed in production ([P3] Supplementary details, the
// hardware-aware prefix scheduler in production; [P1] 4.2.5 and 8.5).  Two
// decisions per round, both on the candidate order of Algorithm 1 (a
// descending, then r, then j ascending; a > 0 only):
//  * admission: the verify batch holds at most K_in tokens, a capacity that
//    was planned two rounds earlier.  The R anchors are always verified, so
//    the min(K_in, N_max) - R best candidates of THIS round are admitted
//    (dynamic top-K; clamped to [0, |E|]); Theta is not consulted.
//  * planning: over THIS round's sorted candidates, the prefix length q* that
//    maximises Theta_q = tau_q * SPS(R + q), q = 0..|E| (global search, no
//    early stop; the first maximum wins; Theta = 0 past N_max), gives the
//    capacity K_plan = R + q* that a round two rounds later admits with.
// Reading: the capacity is counted in verify tokens, anchors included (the
// pages call it the batch capacity); it is handed over as that token count.
// tau and Theta are computed as in Algorithm 1 (2^-32 fixed point, one double
// product).
// Out: ell [R]; a [R][gamma] (nullable); N = sum(1 + ell); Theta of the
//      admitted schedule; K_plan; Theta_{q*}.
int orc_async_schedule(int R, int gamma, const float* c, const double* sps, int N_max, int K_in,
                       int32_t* ell, float* a_out, int32_t* N_out, double* theta,
                       int32_t* K_plan, double* theta_plan) {
    if (R < 0 || gamma < 1 || N_max < R) return 1;
    std::vector<float> a((size_t)R * gamma);
    for (int r = 0; r < R; ++r) {
        float acc = 1.0f;
        for (int j = 1; j <= gamma; ++j) {
            acc = acc * c[(int64_t)r * gamma + (j - 1)];   // float32 product
            a[(size_t)r * gamma + (j - 1)] = acc;
        }
    }
    if (a_out) std::memcpy(a_out, a.data(), a.size() * sizeof(float));
    struct Cand { float a; int r; int j; };
    std::vector<Cand> E;
    for (int r = 0; r < R; ++r)
        for (int j = 1; j <= gamma; ++j) {
            const float av = a[(size_t)r * gamma + (j - 1)];
            if (av > 0.0f) E.push_back({av, r, j});
        }
    std::sort(E.begin(), E.end(), [](const Cand& p, const Cand& q) {
        if (p.a != q.a) return p.a > q.a;
        if (p.r != q.r) return p.r < q.r;
        return p.j < q.j;
    });
    auto fix = [](float av) -> int64_t { return (int64_t)std::llrint((double)av * 0x1p32); };
    auto theta_of = [&](int64_t tau_fx, int64_t B) -> double {
        if (B > N_max) return 0.0;
        return ((double)tau_fx * 0x1p-32) * sps[B];
    };
    // tau_q for every prefix length q = 0..|E|
    std::vector<int64_t> tau(E.size() + 1);
    tau[0] = (int64_t)R << 32;
    for (size_t q = 0; q < E.size(); ++q) tau[q + 1] = tau[q] + fix(E[q].a);

    // admission: the best K_in - R candidates
    const int64_t cap = std::min<int64_t>(K_in, N_max);
    const int64_t take = std::max<int64_t>(0, std::min<int64_t>(cap - R, (int64_t)E.size()));
    for (int r = 0; r < R; ++r) ell[r] = 0;
    for (int64_t q = 0; q < take; ++q) ell[E[q].r] = std::max(ell[E[q].r], E[q].j);
    int64_t N = 0;
    for (int r = 0; r < R; ++r) N += 1 + ell[r];
    if (N_out) *N_out = (int32_t)N;
    if (theta) *theta = theta_of(tau[take], R + take);

    // planning: global search over all prefix lengths
    size_t qbest = 0;
    double best = theta_of(tau[0], R);
    for (size_t q = 1; q <= E.size(); ++q) {
        const double th = theta_of(tau[q], R + (int64_t)q);
        if (th > best) { best = th; qbest = q; }
    }
    if (K_plan) *K_plan = R + (int32_t)qbest;
    if (theta_plan) *theta_plan = best;
    return 0;
}

// ----------------------------------------------------------------- pack ---
// Ragged pack ([P3] Supplementary details, variable-length routing; [P4] 3.3):
// all requests' tokens flattened as independent elements with an offset array
// and per-token marker tensors (owning request, position inside the block).
// Slots past N (capacity R*width) are padded with -1.
void orc_pack(int R, int width, const int32_t* rows, const int32_t* len, int32_t* cu,
              int32_t* flat, int32_t* marker_req, int32_t* marker_pos, int32_t* N_out) {
    cu[0] = 0;
    for (int r = 0; r < R; ++r) cu[r + 1] = cu[r] + len[r];
    const int64_t cap = (int64_t)R * width;
    for (int64_t q = 0; q < cap; ++q) {
        flat[q] = -1;
        if (marker_req) marker_req[q] = -1;
        if (marker_pos) marker_pos[q] = -1;
    }
    for (int r = 0; r < R; ++r)
        for (int j = 0; j < len[r]; ++j) {
            const int64_t q = cu[r] + j;
            flat[q] = rows[(int64_t)r * width + j];
            if (marker_req) marker_req[q] = r;
            if (marker_pos) marker_pos[q] = j;
        }
    if (N_out) *N_out = cu[R];
}

// --------------------------------------------------------------- verify ---
// Lossless rejection-sampling verification ([P3] Background: accept x_k with
// probability min(1, p_t(x_k)/p_d(x_k)), left to right, the first rejection
// drops the rest; [P1] 2.2: residual resample at the first rejection from
// norm(max(0, p_t - p_d)), bonus token from the next target distribution when
// all are accepted, tau = m + 1, greedy reduction at T = 0).
//  ell [R] scheduled lengths; target rows: verify row j of request i (input
//  token x_j, distribution p_t^{j+1}) sits at row cu[i]+j (layout 0, packed
//  [N][V]) or i*(gamma+1)+j (layout 1, dense [R][gamma+1][V]).
//  x [R][gamma+1]; logp_d, lse_d [R][gamma] (the draft's outputs).
//  U, W1, W2t as in the draft (used to rebuild p_d at a rejected position).
//  force_m [R] nullable; entries >= 0 force the accepted count (lock-step).
//  feat [R][gamma][rank] nullable: bias features of each position (the RNN
//  head's e_k); when given they replace W1[x_{k-1}] in rebuilding p_d.
// Out: m, tau [R]; emitted [R][gamma+1] (-1 past tau); next_anchor [R];
//      logp_t [R][gamma] (log p_t(x_k) for k <= ell, else 0; 0 when T == 0);
//      margin [R] (smallest decision margin of the request).
// Accept test: log u < log p_t(x_k) - log p_d(x_k) with u from the ACCEPT tag.
int orc_verify(int R, int gamma, int64_t V, int rank, double T, uint64_t seed, uint64_t round,
               const int32_t* ell, const int32_t* cu, const float* target, int layout,
               const int32_t* x, const double* logp_d, const double* lse_d,
               const float* U, const float* W1, const float* W2t,
               const int32_t* req_ids, const int32_t* force_m,
               int32_t* m_out, int32_t* tau_out, int32_t* emitted, int32_t* next_anchor,
               double* logp_t, double* margin, const float* feat) {
    if (R < 0 || gamma < 1 || V < 1 || !(T >= 0.0)) return 1;
    std::vector<double> lt(V), s(V), q(V), sc(V);
    for (int i = 0; i < R; ++i) {
        const uint32_t rid = req_ids ? (uint32_t)req_ids[i] : (uint32_t)i;
        const int L = ell[i];
        if (L < 0 || L > gamma) return 2;
        auto row = [&](int j) -> const float* {
            const int64_t rr = (layout == 0) ? (int64_t)cu[i] + j : (int64_t)i * (gamma + 1) + j;
            return target + rr * V;
        };
        const int32_t* xi = x + (int64_t)i * (gamma + 1);
        const int fm = force_m ? force_m[i] : -1;
        double mg = POS_INF;
        int m = L;
        bool rejected = false;
        int64_t y = -1;
        for (int k = 1; k <= gamma; ++k) if (logp_t) logp_t[(int64_t)i * gamma + (k - 1)] = 0.0;
        if (T > 0.0) {
            std::vector<double> lse_t(L + 1);
            for (int j = 0; j <= L; ++j) {
                const float* t = row(j);
                for (int64_t v = 0; v < V; ++v) lt[v] = (double)t[v] / T;
                lse_t[j] = logsumexp(lt.data(), V);
                if (j >= 1 && logp_t)
                    logp_t[(int64_t)i * gamma + (j - 1)] = (double)row(j - 1)[xi[j]] / T - lse_t[j - 1];
            }
            for (int k = 1; k <= L; ++k) {
                const double lpt = (double)row(k - 1)[xi[k]] / T - lse_t[k - 1];
                const double lhs = std::log(uniform01(stream_word(seed, round, TAG_ACCEPT, rid,
                                                                  (uint32_t)k, 0u)));
                const double rhs = lpt - logp_d[(int64_t)i * gamma + (k - 1)];
                mg = std::min(mg, std::fabs(lhs - rhs));
                bool accept = (float)lhs < (float)rhs;
                if (fm >= 0) accept = (k <= fm);
                if (!accept) { m = k - 1; rejected = true; break; }
            }
            double mc = POS_INF;
            if (rejected) {
                const int k = m + 1;
                const float* t = row(k - 1);
                for (int64_t v = 0; v < V; ++v) lt[v] = (double)t[v] / T;
                if (feat) {
                    // the draft's bias features of this position (RNN head)
                    const float* e = feat + ((int64_t)i * gamma + (k - 1)) * rank;
                    const float* Uk = U + ((int64_t)i * gamma + (k - 1)) * V;
                    for (int64_t v = 0; v < V; ++v) {
                        double b = 0.0;
                        for (int j = 0; j < rank; ++j) b += (double)e[j] * (double)W2t[v * rank + j];
                        s[v] = (double)Uk[v] + b;
                    }
                } else {
                    markov_scores(V, rank, U + ((int64_t)i * gamma + (k - 1)) * V, W1, W2t,
                                  xi[k - 1], s.data());
                }
                for (int64_t v = 0; v < V; ++v) s[v] /= T;
                const double tot = residual_weights(V, lt.data(), lse_t[k - 1], s.data(),
                                                    lse_d[(int64_t)i * gamma + (k - 1)], q.data());
                if (tot > 0.0) {
                    for (int64_t v = 0; v < V; ++v) sc[v] = q[v] > 0.0 ? std::log(q[v]) : NEG_INF;
                    y = cgm_sample(sc.data(), V, seed, round, TAG_RESID_CHUNK, TAG_RESID_ELEM,
                                   rid, (uint32_t)k, &mc);
                } else {
                    y = cgm_sample(lt.data(), V, seed, round, TAG_RESID_CHUNK, TAG_RESID_ELEM,
                                   rid, (uint32_t)k, &mc);
                }
            } else {
                const float* t = row(L);
                for (int64_t v = 0; v < V; ++v) lt[v] = (double)t[v] / T;
                y = cgm_sample(lt.data(), V, seed, round, TAG_BONUS_CHUNK, TAG_BONUS_ELEM,
                               rid, (uint32_t)(L + 1), &mc);
            }
            mg = std::min(mg, mc);
        } else {
            for (int k = 1; k <= L; ++k) {
                const float* t = row(k - 1);
                for (int64_t v = 0; v < V; ++v) lt[v] = (double)t[v];
                double g;
                const int64_t am = argmax_f32_decision(lt.data(), V, &g);
                mg = std::min(mg, g);
                bool accept = (xi[k] == am);
                if (fm >= 0) accept = (k <= fm);
                if (!accept) { m = k - 1; rejected = true; y = am; break; }
            }
            if (!rejected || fm >= 0) {
                const int j = rejected ? m : L;
                const float* t = row(j);
                for (int64_t v = 0; v < V; ++v) lt[v] = (double)t[v];
                double g;
                y = argmax_f32_decision(lt.data(), V, &g);
                mg = std::min(mg, g);
            }
        }
        m_out[i] = m;
        tau_out[i] = m + 1;
        int32_t* em = emitted + (int64_t)i * (gamma + 1);
        for (int q2 = 0; q2 <= gamma; ++q2) em[q2] = -1;
        for (int q2 = 0; q2 < m; ++q2) em[q2] = xi[q2 + 1];
        em[m] = (int32_t)y;
        next_anchor[i] = (int32_t)y;
        if (margin) margin[i] = mg;
    }
    return 0;
}

// ------------------------------------------- single-step acceptance rate ---
// The confidence head's supervision target ([P3] Method details, confidence
// head): c*_k = 1 - TV(p_d^k, p_t^k) = sum_v min(p_d^k(v), p_t^k(v)), the
// probability that the rejection test accepts position k given the prefix.
// For every request i and k = 1..gamma: p_d^k is the tempered draft
// distribution of position k given x_{k-1} (scores (U_k + W1[x_{k-1}] W2) / T,
// normalised here), p_t^k = softmax(row / T) of the dense target row
// i*(gamma+1) + k-1 (verify row k-1, input x_{k-1}).
// T == 0 (point masses): c*_k = 1 if x_k (the greedy draft's pick) is the first
// argmax of the target row, else 0; the argmax is decided on float32 values
// and its gap is the margin.
// Out: c_star [R][gamma]; margin [R][gamma] (nullable; +inf when T > 0).
int orc_acceptance_rate(int R, int gamma, int64_t V, int rank, double T, const float* target,
                        const int32_t* x, const float* U, const float* W1, const float* W2t,
                        double* c_star, double* margin, const float* feat) {
    if (R < 0 || gamma < 1 || V < 1 || !(T >= 0.0)) return 1;
    std::vector<double> s(V), lt(V);
    for (int i = 0; i < R; ++i) {
        const int32_t* xi = x + (int64_t)i * (gamma + 1);
        for (int k = 1; k <= gamma; ++k) {
            const float* t = target + ((int64_t)i * (gamma + 1) + (k - 1)) * V;
            double cs, mg = POS_INF;
            if (T > 0.0) {
                if (feat) {
                    // the draft's bias features of this position (RNN head)
                    const float* e = feat + ((int64_t)i * gamma + (k - 1)) * rank;
                    const float* Uk = U + ((int64_t)i * gamma + (k - 1)) * V;
                    for (int64_t v = 0; v < V; ++v) {
                        double b = 0.0;
                        for (int j = 0; j < rank; ++j) b += (double)e[j] * (double)W2t[v * rank + j];
                        s[v] = (double)Uk[v] + b;
                    }
                } else {
                    markov_scores(V, rank, U + ((int64_t)i * gamma + (k - 1)) * V, W1, W2t,
                                  xi[k - 1], s.data());
                }
                for (int64_t v = 0; v < V; ++v) { s[v] /= T; lt[v] = (double)t[v] / T; }
                const double lse_d = logsumexp(s.data(), V);
                const double lse_t = logsumexp(lt.data(), V);
                cs = 0.0;
                for (int64_t v = 0; v < V; ++v)
                    cs += std::min(std::exp(s[v] - lse_d), std::exp(lt[v] - lse_t));
            } else {
                for (int64_t v = 0; v < V; ++v) lt[v] = (double)t[v];
                const int64_t am = argmax_f32_decision(lt.data(), V, &mg);
                cs = (xi[k] == am) ? 1.0 : 0.0;
            }
            c_star[(int64_t)i * gamma + (k - 1)] = cs;
            if (margin) margin[(int64_t)i * gamma + (k - 1)] = mg;
        }
    }
    return 0;
}

// ------------------------------------------------------------- STS fit ---
// Sequential temperature scaling ([P3] Method details, post-hoc calibration;
// [P1] 4.2.3).  Held-out data: n blocks with raw confidence logits z [n][gamma]
// (c_k = sigmoid(z_k / t_k)) and the number m [n] of drafts the target
// accepted; the label of position k is "the prefix 1..k was accepted",
// y_k = [m >= k].  Left to right, k = 1..gamma, earlier temperatures fixed:
// for every candidate t of the grid (in its order),
//   A_k(t) = A_{k-1} * sigmoid(z_k / t)          (A_0 = 1; cumulative product)
//   ECE(t) = (1/n) sum_b | sum_{i in bin b} (A_k,i - y_k,i) |
// over nbins equal-width bins of [0, 1], bin = min(floor(A nbins), nbins - 1)
// (the expected calibration error: bin weight n_b/n times |mean A - mean y|);
// t_k = the first grid value with the smallest ECE.  All in double.
// force_t (nullable, [gamma]): entries > 0 replace the chosen temperature
// (lock-step checking); the ECE reported is then that of the forced value.
// Out: t [gamma] (float, the grid's value); ece [gamma]; margin [gamma] = the
// smaller of (second-smallest ECE - smallest ECE) and the closest distance of
// any A nbins to a bin edge (both nullable-safe: margin may be null).
int orc_sts_fit(int n, int gamma, const float* z, const int32_t* m, const float* grid, int G,
                int nbins, const float* force_t, float* t_out, double* ece_out, double* margin) {
    if (n < 1 || gamma < 1 || G < 1 || nbins < 1) return 1;
    std::vector<double> A(n, 1.0), Ak(n), d(nbins);
    for (int k = 1; k <= gamma; ++k) {
        double best = POS_INF, second = POS_INF, edge = POS_INF;
        int gbest = 0;
        std::vector<double> eces(G);
        for (int g = 0; g < G; ++g) {
            const double t = (double)grid[g];
            std::fill(d.begin(), d.end(), 0.0);
            for (int i = 0; i < n; ++i) {
                const double c = 1.0 / (1.0 + std::exp(-(double)z[(int64_t)i * gamma + (k - 1)] / t));
                const double a = A[i] * c;
                const double pos = a * nbins;
                int b = (int)std::floor(pos);
                if (b > nbins - 1) b = nbins - 1;
                if (b < 0) b = 0;
                edge = std::min(edge, std::fabs(pos - std::nearbyint(pos)));
                d[b] += a - (m[i] >= k ? 1.0 : 0.0);
            }
            double e = 0.0;
            for (int b = 0; b < nbins; ++b) e += std::fabs(d[b]);
            e /= n;
            eces[g] = e;
            if (e < best) { second = best; best = e; gbest = g; }
            else if (e < second) second = e;
        }
        if (force_t && force_t[k - 1] > 0.0f) {
            for (int g = 0; g < G; ++g) if (grid[g] == force_t[k - 1]) { gbest = g; break; }
        }
        const double t = (double)grid[gbest];
        for (int i = 0; i < n; ++i)
            A[i] *= 1.0 / (1.0 + std::exp(-(double)z[(int64_t)i * gamma + (k - 1)] / t));
        t_out[k - 1] = grid[gbest];
        if (ece_out) ece_out[k - 1] = eces[gbest];
        if (margin) margin[k - 1] = std::min(second - best, edge);
    }
    return 0;
}

}  // extern "C"
