// Host-sanitizer driver for the CPU oracle (test infrastructure).  Built
// together with oracle.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_oracle_sanitizers.py, it calls
// every exported oracle function on small shapes with fixed pseudo-random
// inputs: both storage modes, MHA and GQA, both lock policies and KL
// directions, the semi-autoregressive and SlowFast samplers, the drift-aware
// refresh of locked positions, commit / lock / counter overrides, a sampled step, and each unit routine.  Any invalid
// access or undefined behaviour aborts with the sanitizer's report; a clean
// run prints "sanitized run ok".
#include <cstdint>
#include <cstdio>
#include <vector>

#include "oracle.cpp"

namespace {

uint64_t g_lcg = 0x9E3779B97F4A7C15ull;
double urand() {  // in [-1, 1)
  g_lcg = g_lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(g_lcg >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
std::vector<float> mat(size_t n, double scale) {
  std::vector<float> v(n);
  for (auto& x : v) x = (float)(urand() * scale);
  return v;
}

int run_model(int nq, int nkv, int bf16, int policy, int sampler, int kl_dir, int refresh = 0) {
  orc_model m{2, 32, nq, nkv, 32 / nq, 48, 40, 39, 10000.0, 1e-5, bf16};
  const int L = m.n_layers, d = m.d_model, hd = m.head_dim, dff = m.d_ff, V = m.vocab;
  const int qkv = (nq + 2 * nkv) * hd;
  orc_run r{};
  r.batch = 2;
  r.seq_len = 24;
  r.prompt_len = 6;
  r.steps = 10;
  r.block_len = 9;
  r.kl_eps = policy ? 1e30 : -1.0;
  r.conf_tau = 0.0;
  r.n_consec = 2;
  r.kl_dir = kl_dir;
  r.lock_prompt_after_first_step = 1;
  r.policy = policy;
  r.sampler = sampler;
  r.sf_k = 2;
  r.sf_kmax = 3;
  r.sf_whist = 2;
  r.sf_tau_conv = 0.0;
  r.sf_tau_high = 0.5;
  r.sf_var = 1.0;
  r.refresh_budget = refresh;
  r.refresh_eps = 1e-6;
  auto emb = mat((size_t)V * d, 0.5), fn = mat(d, 1.0), lm = mat((size_t)V * d, 0.2);
  std::vector<std::vector<float>> an(L), wq(L), wo(L), ff(L), wg(L), wu(L), wd(L);
  std::vector<const float*> pan(L), pwq(L), pwo(L), pff(L), pwg(L), pwu(L), pwd(L);
  for (int l = 0; l < L; ++l) {
    an[l] = mat(d, 1.0); wq[l] = mat((size_t)qkv * d, 0.1); wo[l] = mat((size_t)d * nq * hd, 0.1);
    ff[l] = mat(d, 1.0); wg[l] = mat((size_t)dff * d, 0.1); wu[l] = mat((size_t)dff * d, 0.1);
    wd[l] = mat((size_t)d * dff, 0.1);
    pan[l] = an[l].data(); pwq[l] = wq[l].data(); pwo[l] = wo[l].data(); pff[l] = ff[l].data();
    pwg[l] = wg[l].data(); pwu[l] = wu[l].data(); pwd[l] = wd[l].data();
  }
  orc_weights w{emb.data(), fn.data(), lm.data(), pan.data(), pwq.data(), pwo.data(),
                pff.data(), pwg.data(), pwu.data(), pwd.data()};
  std::vector<int32_t> prompt(r.batch * r.prompt_len);
  for (size_t i = 0; i < prompt.size(); ++i) prompt[i] = (int32_t)(i * 7 % (V - 1));
  orc_state* s = orc_create(&m, &w, &r, prompt.data());
  if (!s) return 1;
  const int BN = r.batch * r.seq_len;
  std::vector<int32_t> tok(BN), cnt(BN), sf(r.batch * 13);
  std::vector<uint8_t> lk(BN), hp(BN), fz(BN), rf(BN);
  std::vector<float> dr(BN);
  for (int t = 0; t < r.steps; ++t) {
    if (orc_step(s) != 0) return 2;
    const int M = orc_m(s);
    std::vector<int32_t> seq(M), pos(M), am(M);
    std::vector<uint8_t> real(M), hk(M);
    std::vector<double> conf(M), kl(M), lse(M);
    orc_get_rows(s, seq.data(), pos.data(), real.data());
    orc_get_stats(s, am.data(), conf.data(), kl.data(), lse.data(), hk.data());
    std::vector<int32_t> rows(orc_n_logit_rows(s));
    std::vector<double> z(rows.size() * (size_t)V);
    orc_get_logits(s, rows.data(), z.data());
    (void)orc_flops(s);
    if (t % 3 == 2 && M > 0) {  // overrides: commit one masked row, lock nothing, reset counters
      orc_get_tokens(s, tok.data());
      std::vector<int32_t> cs, cp, ct;
      for (int i = 0; i < M; ++i)
        if (tok[(size_t)seq[i] * r.seq_len + pos[i]] == m.mask_id) {
          cs.push_back(seq[i]); cp.push_back(pos[i]); ct.push_back(am[i]);
          break;
        }
      std::vector<uint8_t> none(BN, 0);
      std::vector<int32_t> zc(BN, 0);
      if (orc_lock_update(s, cs.data(), cp.data(), ct.data(), (int)cs.size(), none.data(),
                          zc.data()) != 0)
        return 3;
    } else if (orc_lock_update(s, nullptr, nullptr, nullptr, -1, nullptr, nullptr) != 0) {
      return 4;
    }
    orc_get_tokens(s, tok.data()); orc_get_locked(s, lk.data()); orc_get_cnt(s, cnt.data());
    orc_get_has_prev(s, hp.data()); orc_get_frozen(s, fz.data()); orc_get_sf(s, sf.data());
    orc_get_drift(s, dr.data()); orc_get_refresh(s, rf.data());
    std::vector<int32_t> c0(orc_n_commits(s)), c1(c0.size()), c2(c0.size());
    orc_get_commits(s, c0.data(), c1.data(), c2.data());
  }
  std::vector<double> kk((size_t)r.batch * nkv * r.seq_len * hd), vv(kk.size());
  for (int l = 0; l < L; ++l) orc_get_kv(s, l, kk.data(), vv.data());
  orc_destroy(s);
  // a sampled step on a fresh run (two rows), followed by a full override
  s = orc_create(&m, &w, &r, prompt.data());
  const int32_t sample[2] = {1, 5};
  if (orc_step_sample(s, sample, 2) != 0) return 5;
  std::vector<uint8_t> none(BN, 0);
  if (orc_lock_update(s, nullptr, nullptr, nullptr, 0, none.data(), nullptr) != 0) return 6;
  orc_destroy(s);
  return 0;
}

int run_units() {
  const int M = 5, d = 16, nh = 2, hd = 8, V = 12, B = 2, N = 7, K = 16, Nout = 9;
  std::vector<double> x(M * d), y(M * d), u(M * nh * hd);
  for (auto& v : x) v = urand();
  for (auto& v : u) v = urand();
  std::vector<float> g = mat(d, 1.0), W = mat((size_t)Nout * K, 0.3);
  orc_unit_rmsnorm(x.data(), g.data(), M, d, 1e-5, y.data());
  std::vector<int32_t> pos = {0, 3, 6, 2, 5};
  orc_unit_rope(u.data(), pos.data(), M, nh, hd, 10000.0);
  std::vector<double> lin((size_t)M * Nout);
  orc_unit_linear(x.data(), W.data(), M, Nout, K, lin.data());
  std::vector<double> q((size_t)M * nh * hd), kc((size_t)B * 1 * N * hd), vc(kc.size()),
      o(q.size());
  for (auto& v : q) v = urand();
  for (auto& v : kc) v = urand();
  for (auto& v : vc) v = urand();
  std::vector<int32_t> rs = {0, 0, 1, 1, 1};
  orc_unit_attention(q.data(), rs.data(), kc.data(), vc.data(), M, B, N, nh, 1, hd, o.data());
  std::vector<double> z((size_t)M * V), prev((size_t)M * V), lse(M), conf(M), kl(M),
      logp((size_t)M * V);
  std::vector<int32_t> am(M);
  std::vector<uint8_t> hpv = {1, 0, 1, 1, 0};
  for (auto& v : z) v = 3 * urand();
  for (auto& v : prev) v = -std::log((double)V) + 0.1 * urand();
  for (int dir = 0; dir < 2; ++dir)
    orc_unit_vocab_stats(z.data(), prev.data(), hpv.data(), M, V, V - 1, dir, lse.data(),
                         am.data(), conf.data(), kl.data(), logp.data());
  orc_run r{};
  r.batch = 1; r.seq_len = 40; r.prompt_len = 4; r.steps = 12; r.block_len = 9;
  r.n_consec = 2; r.policy = 1; r.kl_eps = 1e-3;
  int32_t out4[4];
  for (int t = 0; t < r.steps; ++t) orc_unit_schedule(&r, t, out4);
  orc_model m{1, 8, 1, 1, 8, 8, V, V - 1, 0.0, 1e-5, 0};
  std::vector<int32_t> lseq = {0, 0, 0}, lpos = {1, 5, 6}, larg = {3, 4, 5};
  std::vector<uint8_t> lreal = {1, 0, 0}, lhk = {1, 1, 0}, locked(r.seq_len, 0);
  std::vector<double> lconf = {0.5, 0.7, 0.2}, lkl = {1e-4, 2e-3, NAN};
  std::vector<int32_t> xx(r.seq_len, V - 1), cn(r.seq_len, 0);
  if (orc_unit_lock_transition(&m, &r, 0, 3, lseq.data(), lpos.data(), lreal.data(),
                               larg.data(), lconf.data(), lkl.data(), lhk.data(), xx.data(),
                               locked.data(), cn.data(), nullptr, nullptr) != 0)
    return 7;
  {  // the same transition with a refresh set and drift
    orc_run rr = r;
    rr.refresh_budget = 2;
    rr.refresh_eps = 1e-3;
    std::vector<uint8_t> rlock(r.seq_len, 0), rsel(r.seq_len, 0);
    std::vector<float> rdrift(r.seq_len, 0.f);
    rlock[1] = rlock[5] = rlock[30] = 1;
    rdrift[5] = 2e-3f;
    rdrift[30] = INFINITY;
    orc_unit_refresh_select(&rr, rlock.data(), rdrift.data(), rsel.data());
    std::vector<int32_t> rcnt(r.seq_len, 0), rx(r.seq_len, V - 1);
    if (orc_unit_lock_transition(&m, &rr, 1, 3, lseq.data(), lpos.data(), lreal.data(),
                                 larg.data(), lconf.data(), lkl.data(), lhk.data(), rx.data(),
                                 rlock.data(), rcnt.data(), rsel.data(), rdrift.data()) != 0)
      return 8;
  }
  std::vector<uint64_t> bits = {0x5ull, 0x3Full, ~0ull, 0ull};  // [2 sequences][2 words]
  std::vector<int32_t> cseq(2 * 70), cpos(2 * 70), mb(2);
  (void)orc_unit_compact(bits.data(), 2, 70, cseq.data(), cpos.data(), mb.data());
  orc_run sr = r;
  sr.sampler = 1; sr.sf_k = 1; sr.sf_kmax = 2; sr.sf_whist = 2; sr.sf_tau_conv = 0.3;
  sr.sf_tau_high = 0.6; sr.sf_var = 1.0;
  std::vector<int32_t> sp = {2, 3, 4, 9, 12}, sa = {1, 2, 3, 4, 5}, state(13, 0), ccp(5), cct(5);
  std::vector<double> sc = {0.5, 0.1, 0.7, 0.35, 0.2};
  std::vector<int32_t> sx(r.seq_len, V - 1);
  std::vector<uint8_t> sfz(r.seq_len, 0), shp(r.seq_len, 1);
  for (int it = 0; it < 4; ++it)
    (void)orc_unit_slowfast(&sr, V - 1, r.seq_len, 5, sp.data(), sa.data(), sc.data(), sx.data(),
                            sfz.data(), shp.data(), state.data(), ccp.data(), cct.data());
  (void)orc_bf16_round(1.0 / 3.0);
  (void)orc_num_threads();
  return 0;
}

}  // namespace

int main() {
  int rc = run_units();
  for (int bf16 = 0; bf16 < 2 && !rc; ++bf16)
    for (int policy = 0; policy < 2 && !rc; ++policy)
      for (int sampler = 0; sampler < 2 && !rc; ++sampler) {
        rc = run_model(4, 4, bf16, policy, sampler, bf16);
        if (!rc) rc = run_model(4, 2, bf16, policy, sampler, 1 - bf16);
      }
  for (int bf16 = 0; bf16 < 2 && !rc; ++bf16) rc = run_model(4, 2, bf16, 1, 0, bf16, 3);
  if (rc) {
    std::printf("driver step failed: %d\n", rc);
    return rc;
  }
  std::printf("sanitized run ok\n");
  return 0;
}
