// Plain fp32 CPU decoder -- TEST INFRASTRUCTURE, not part of the product.
//
// Only the tests, the smoke check and the benchmark's CPU-baseline leg load
// this library.  It shares no code with the GPU path.  It computes the batch-1
// greedy decode loop of a ~2B FP16 decoder without speculative decoding
// (revietech.ru, "Kog vyzhimayet maksimum iz GPU: 3000 tokenov/s", section
// "Chto takoye monokernel"; remio.ai, "Kog stawia na glebsza optymalizacje
// GPU...", section "Dlaczego Kog idzie glebiej w wnioskowanie GPU"), read as
// the same standard dense pre-norm decoder as the float64 oracle in
// decoder.py, written out again independently: per layer RMSNorm, the q/k/v
// projections, rotary position embedding, the key/value cache append,
// causal grouped-query attention over the cache, the output projection and
// residual, RMSNorm, the SwiGLU feed-forward block and residual; then the final
// RMSNorm, the LM head and the greedy argmax (the lowest index on ties).
//
// Everything is fp32 with one plain loop per operation, in the order written
// above.  There is no blocking and no fusion.  The one concession to time is
// that each matrix-vector product splits its output rows over std::thread
// workers; each row is still one sequential fp32 sum over its columns, so the
// thread count does not change any result.  Rotation angles are computed in
// double and rounded to fp32, because an fp32 angle of a position in the
// thousands is off by about 1e-3 radians.
//
// Weights are row-major fp32 arrays ([rows][cols], the 16-bit stored values
// widened exactly).  The library borrows them: the caller keeps them alive for
// the decoder's lifetime.  The key/value cache is fp32 and owned by the
// decoder.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <new>
#include <thread>
#include <vector>

extern "C" {

struct oc_shape {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab;
  float rms_eps, rope_base;
};

struct oc_layer {
  const float *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
};

struct oc_weights {
  const float* tok_emb;     // [vocab][d_model]
  const float* final_norm;  // [d_model]
  const float* lm_head;     // [vocab][d_model]
  const oc_layer* layers;   // [n_layers], copied at creation
};

}  // extern "C"

namespace {

struct Decoder {
  oc_shape s;
  const float* emb;
  const float* fnorm;
  const float* lm;
  std::vector<oc_layer> layers;
  int max_seq, n_threads, pos = 0;
  // cache[l] K then V: [n_kv_heads][max_seq][head_dim] each
  std::vector<std::vector<float>> kc, vc;
};

// y[r] = sum_c W[r][c] x[c] for r in [0, rows), rows split over threads.
void matvec(const float* W, const float* x, float* y, int rows, int cols, int n_threads) {
  auto part = [&](int r0, int r1) {
    for (int r = r0; r < r1; ++r) {
      const float* w = W + (size_t)r * cols;
      float acc = 0.f;
      for (int c = 0; c < cols; ++c) acc += w[c] * x[c];
      y[r] = acc;
    }
  };
  const int T = n_threads < 1 ? 1 : (n_threads > rows ? rows : n_threads);
  if (T <= 1) {
    part(0, rows);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(T);
  for (int i = 0; i < T; ++i) {
    const int r0 = (int)((int64_t)rows * i / T), r1 = (int)((int64_t)rows * (i + 1) / T);
    pool.emplace_back(part, r0, r1);
  }
  for (auto& th : pool) th.join();
}

// out = x / sqrt(mean(x^2) + eps) * g
void rmsnorm(const float* x, const float* g, float* out, int n, float eps) {
  float ss = 0.f;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  const float r = 1.f / sqrtf(ss / (float)n + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * r * g[i];
}

// Rotate the pairs (i, i + hd/2) of one head's vector by pos * base^(-2i/hd).
void rotate(float* v, int hd, int pos, float base) {
  const int half = hd / 2;
  for (int i = 0; i < half; ++i) {
    const double ang = (double)pos * pow((double)base, -2.0 * i / hd);
    const float c = (float)cos(ang), sn = (float)sin(ang);
    const float a = v[i], b = v[i + half];
    v[i] = a * c - b * sn;
    v[i + half] = a * sn + b * c;
  }
}

// Feed token `tok` at position d.pos; logits (vocab floats) may be null.
// Returns the greedy token.
int step(Decoder& d, int tok, float* logits) {
  const oc_shape& s = d.s;
  const int D = s.d_model, hd = s.head_dim, hq = s.n_heads, hkv = s.n_kv_heads, F = s.d_ffn;
  const int group = hq / hkv, pos = d.pos;
  std::vector<float> x(d.emb + (size_t)tok * D, d.emb + (size_t)(tok + 1) * D);
  std::vector<float> xn(D), q(hq * hd), k(hkv * hd), v(hkv * hd), att(hq * hd), proj(D), g(F), u(F), h(F);
  std::vector<float> sc(pos + 1);
  const float scale = 1.f / sqrtf((float)hd);
  for (int l = 0; l < s.n_layers; ++l) {
    const oc_layer& w = d.layers[l];
    rmsnorm(x.data(), w.attn_norm, xn.data(), D, s.rms_eps);
    matvec(w.wq, xn.data(), q.data(), hq * hd, D, d.n_threads);
    matvec(w.wk, xn.data(), k.data(), hkv * hd, D, d.n_threads);
    matvec(w.wv, xn.data(), v.data(), hkv * hd, D, d.n_threads);
    for (int hh = 0; hh < hq; ++hh) rotate(q.data() + hh * hd, hd, pos, s.rope_base);
    for (int hh = 0; hh < hkv; ++hh) rotate(k.data() + hh * hd, hd, pos, s.rope_base);
    for (int hh = 0; hh < hkv; ++hh) {
      memcpy(&d.kc[l][((size_t)hh * d.max_seq + pos) * hd], k.data() + hh * hd, hd * sizeof(float));
      memcpy(&d.vc[l][((size_t)hh * d.max_seq + pos) * hd], v.data() + hh * hd, hd * sizeof(float));
    }
    // causal attention: query head hh reads cache head hh / group, keys 0 .. pos
    for (int hh = 0; hh < hq; ++hh) {
      const float* qh = q.data() + hh * hd;
      const float* K = &d.kc[l][(size_t)(hh / group) * d.max_seq * hd];
      const float* V = &d.vc[l][(size_t)(hh / group) * d.max_seq * hd];
      float m = -INFINITY;
      for (int j = 0; j <= pos; ++j) {
        float dot = 0.f;
        for (int e = 0; e < hd; ++e) dot += qh[e] * K[(size_t)j * hd + e];
        sc[j] = dot * scale;
        if (sc[j] > m) m = sc[j];
      }
      float z = 0.f;
      for (int j = 0; j <= pos; ++j) {
        sc[j] = expf(sc[j] - m);
        z += sc[j];
      }
      float* o = att.data() + hh * hd;
      for (int e = 0; e < hd; ++e) o[e] = 0.f;
      for (int j = 0; j <= pos; ++j) {
        const float p = sc[j] / z;
        for (int e = 0; e < hd; ++e) o[e] += p * V[(size_t)j * hd + e];
      }
    }
    matvec(w.wo, att.data(), proj.data(), D, hq * hd, d.n_threads);
    for (int i = 0; i < D; ++i) x[i] += proj[i];
    rmsnorm(x.data(), w.ffn_norm, xn.data(), D, s.rms_eps);
    matvec(w.w_gate, xn.data(), g.data(), F, D, d.n_threads);
    matvec(w.w_up, xn.data(), u.data(), F, D, d.n_threads);
    for (int i = 0; i < F; ++i) h[i] = g[i] / (1.f + expf(-g[i])) * u[i];
    matvec(w.w_down, h.data(), proj.data(), D, F, d.n_threads);
    for (int i = 0; i < D; ++i) x[i] += proj[i];
  }
  rmsnorm(x.data(), d.fnorm, xn.data(), D, s.rms_eps);
  std::vector<float> lg(s.vocab);
  matvec(d.lm, xn.data(), lg.data(), s.vocab, D, d.n_threads);
  int best = 0;
  for (int i = 1; i < s.vocab; ++i)
    if (lg[i] > lg[best]) best = i;
  if (logits) memcpy(logits, lg.data(), lg.size() * sizeof(float));
  d.pos = pos + 1;
  return best;
}

}  // namespace

extern "C" {

// A decoder for up to max_seq positions using n_threads workers per
// matrix-vector product.  Returns null on invalid arguments or when out of
// memory.
void* oc_create(const oc_shape* s, const oc_weights* w, int32_t max_seq, int32_t n_threads) {
  if (!s || !w || !w->tok_emb || !w->final_norm || !w->lm_head || !w->layers || max_seq < 1) return nullptr;
  if (s->n_layers < 1 || s->d_model < 1 || s->n_heads < 1 || s->n_kv_heads < 1 || s->head_dim < 2 ||
      s->head_dim % 2 || s->n_heads % s->n_kv_heads || s->d_ffn < 1 || s->vocab < 1)
    return nullptr;
  Decoder* d = new (std::nothrow) Decoder();
  if (!d) return nullptr;
  try {
    d->s = *s;
    d->emb = w->tok_emb;
    d->fnorm = w->final_norm;
    d->lm = w->lm_head;
    d->layers.assign(w->layers, w->layers + s->n_layers);
    d->max_seq = max_seq;
    d->n_threads = n_threads < 1 ? 1 : n_threads;
    const size_t per = (size_t)s->n_kv_heads * max_seq * s->head_dim;
    d->kc.assign(s->n_layers, std::vector<float>(per, 0.f));
    d->vc.assign(s->n_layers, std::vector<float>(per, 0.f));
  } catch (...) {
    delete d;
    return nullptr;
  }
  return d;
}

void oc_destroy(void* h) { delete static_cast<Decoder*>(h); }

// Replace the cache with n_pos positions of k, v [n_layers][n_kv_heads][n_pos][head_dim]
// (rotated keys); the next step runs at position n_pos.  Returns 0, or -1 on
// invalid arguments.
int32_t oc_set_cache(void* h, const float* k, const float* v, int32_t n_pos) {
  Decoder* d = static_cast<Decoder*>(h);
  if (!d || n_pos < 0 || n_pos >= d->max_seq || (n_pos > 0 && (!k || !v))) return -1;
  const oc_shape& s = d->s;
  for (int l = 0; l < s.n_layers; ++l)
    for (int hh = 0; hh < s.n_kv_heads; ++hh)
      for (int p = 0; p < n_pos; ++p) {
        const size_t src = (((size_t)l * s.n_kv_heads + hh) * n_pos + p) * s.head_dim;
        const size_t dst = ((size_t)hh * d->max_seq + p) * s.head_dim;
        memcpy(&d->kc[l][dst], k + src, s.head_dim * sizeof(float));
        memcpy(&d->vc[l][dst], v + src, s.head_dim * sizeof(float));
      }
  d->pos = n_pos;
  return 0;
}

// Feed one token; writes vocab logits when `logits` is not null and returns the
// greedy token, or -1 when the cache is full or the token is out of range.
int32_t oc_step(void* h, int32_t token, float* logits) {
  Decoder* d = static_cast<Decoder*>(h);
  if (!d || d->pos >= d->max_seq || token < 0 || token >= d->s.vocab) return -1;
  return step(*d, token, logits);
}

int32_t oc_position(const void* h) { return h ? static_cast<const Decoder*>(h)->pos : -1; }

}  // extern "C"
