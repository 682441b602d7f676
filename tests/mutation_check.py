"""Mutation check of the oracle's pins (CPU only, not collected by pytest).

Plants one mistake at a time in a copy of the oracle -- the C arithmetic
(reduction, Adam, constants, 16-bit encode and decode) and the Python layout
code (plan, flatten, memory and volume counts, reshard) -- rebuilds it, and
runs tests/test_oracle_pins.py against it.  A mutant that passes every pin is
a hole in the pins.  Nothing outside the given work directory is modified.

    python tests/mutation_check.py WORKDIR [substring ...]

takes about 30 s per mutant (the exhaustive cast checks dominate).
"""
import os, shutil, subprocess, sys, time
R = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BASE = None
C = 'oracle/zero_oracle.c'
P = 'oracle/__init__.py'
RUN = 'oracle/runner.py'
MUTANTS = [
    # (name, file, old, new)
    ("reduce: start from +0", C, "float acc = orc_widen(slices[0], dt, j);\n        for (int32_t q = 1;", "float acc = 0.0f;\n        for (int32_t q = 0;"),
    ("reduce: reverse rank order", C, "for (int32_t q = 1; q < n_ranks; ++q) {\n            float gq = orc_widen(slices[q], dt, j);", "for (int32_t q = 1; q < n_ranks; ++q) {\n            float gq = orc_widen(slices[n_ranks - q], dt, j);"),
    ("reduce: no grad_scale", C, "float g = acc * grad_scale;", "float g = acc;"),
    ("reduce: skip last rank", C, "for (int32_t q = 1; q < n_ranks; ++q) {", "for (int32_t q = 1; q < n_ranks - 1; ++q) {"),
    ("adam: m keeps g", C, "float m_keep = b1 * m[j];", "float m_keep = b1 * g;"),
    ("adam: c1/c2 swapped", C, "const float b1 = c[0], c1 = c[1], b2 = c[2], c2 = c[3];", "const float b1 = c[0], c1 = c[3], b2 = c[2], c2 = c[1];"),
    ("adam: no m bias correction", C, "float mhat = mn / bc1;", "float mhat = mn;"),
    ("adam: no v bias correction", C, "float vhat = vn / bc2;", "float vhat = vn;"),
    ("adam: eps inside sqrt", C, "float root = sqrtf(vhat);\n        float den = root + eps;", "float root = sqrtf(vhat + eps);\n        float den = root;"),
    ("adam: wrong sign", C, "float wn = w[j] - delta;", "float wn = w[j] + delta;"),
    ("adam: v uses g", C, "float v_new_part = c2 * gsq;", "float v_new_part = c2 * g;"),
    ("adam: fused m update", C, "float mn = m_keep + m_new_part;", "float mn = fmaf(b1, m[j], m_new_part);"),
    ("adam: param from old w", C, "        float wn = w[j] - delta;\n        m[j] = mn;\n        v[j] = vn;\n        w[j] = wn;\n        if (p) p[j] = pdt == ORC_F16 ? orc_f32_to_f16(wn) : orc_f32_to_bf16(wn);", "        float wn = w[j] - delta;\n        float w_old = w[j];\n        m[j] = mn;\n        v[j] = vn;\n        w[j] = wn;\n        if (p) p[j] = pdt == ORC_F16 ? orc_f32_to_f16(w_old) : orc_f32_to_bf16(w_old);"),
    ("adam: fused v update", C, "float vn = v_keep + v_new_part;", "float vn = fmaf(b2, v[j], v_new_part);"),
    ("adam: fused w update", C, "float wn = w[j] - delta;", "float wn = fmaf(-lr, ratio, w[j]);"),
    ("adam: state not stored (m)", C, "        m[j] = mn;\n", "        m[j] = m[j] * 1.0f + 0.0f * mn;\n"),
    ("adam: lr applied twice", C, "float delta = lr * ratio;", "float delta = lr * (lr * ratio);"),
    ("consts: no power in bc1", C, "out[4] = (float)(1.0 - pow(beta1, (double)t));", "out[4] = (float)(1.0 - beta1);"),
    ("consts: bc2 uses beta1", C, "out[5] = (float)(1.0 - pow(beta2, (double)t));", "out[5] = (float)(1.0 - pow(beta1, (double)t));"),
    ("consts: 1-beta1 rounded twice", C, "out[1] = (float)(1.0 - beta1);", "out[1] = 1.0f - (float)beta1;"),
    ("consts: t-1", C, "out[4] = (float)(1.0 - pow(beta1, (double)t));", "out[4] = (float)(1.0 - pow(beta1, (double)(t + 1)));"),
    ("cast: truncate", C, "double r = rint(ax / quantum) * quantum;", "double r = trunc(ax / quantum) * quantum;"),
    ("cast: ties away", C, "double r = rint(ax / quantum) * quantum;", "double r = round(ax / quantum) * quantum;"),
    ("cast: fp16 max off", C, "double maxval = 65504.0;", "double maxval = 65536.0;"),
    ("cast: bf16 NaN pattern", C, "return (uint16_t)((sign << 15) | 0x7fc0);", "return (uint16_t)((sign << 15) | 0x7f80);"),
    ("cast: fp16 subnormal quantum", C, "if (e < emin) e = emin;", "if (e < emin - 1) e = emin - 1;"),
    ("decode: f16 subnormal scale", C, "else if (e == 0) mag = ldexp((double)f, -24);", "else if (e == 0) mag = ldexp((double)f, -25);"),
    ("decode: bf16 exponent bias", C, "else mag = ldexp((double)(128 + f), e - 134);", "else mag = ldexp((double)(128 + f), e - 133);"),
    ("plan: align ignored", P, "    unit = n_d * align\n", "    unit = n_d\n"),
    ("plan: cap rule >=", P, "if bucket_cap > 0 and cur and cur_n + n > bucket_cap:", "if bucket_cap > 0 and cur and cur_n + n >= bucket_cap:"),
    ("plan: reversed rank blocks", P, "        lo = bk.flat_off + rank * bk.shard_numel\n", "        lo = bk.flat_off + (self.n_d - 1 - rank) * bk.shard_numel\n"),
    ("plan: pad at front", P, "            p.tensor_off[t] = flat + numel\n", "            p.tensor_off[t] = flat + numel + (((sum(sizes[u] for u in g) + unit - 1) // unit) * unit - sum(sizes[u] for u in g))\n"),
    ("flatten: pads not zero", P, "    out = np.zeros(p.psi_pad, dtype=dtype)\n", "    out = np.ones(p.psi_pad, dtype=dtype)\n"),
    ("memory: K=16", P, "def memory_closed_form(psi: float, n_d: int, k: int = 12) -> dict:", "def memory_closed_form(psi: float, n_d: int, k: int = 16) -> dict:"),
    ("memory: stage 2 grads full", P, '    "os_g": {"optim", "grads"},', '    "os_g": {"optim"},'),
    ("volume: stage 3 one gather", P, '        ops = {"reduce_scatter": walk(), "all_gather_fwd": walk(), "all_gather_bwd": walk()}', '        ops = {"reduce_scatter": walk(), "all_gather_fwd": walk()}'),
    ("volume: self slice dropped", P, "                total += hi - lo\n", "                total += (hi - lo) if r != perspective else 0\n"),
    ("reshard: source rank 0 only", P, "    full = gather_pack(src, src_shards)\n", "    full = gather_pack(src, [src_shards[0]] * len(src_shards))\n"),
    ("stage3: gather after the step", RUN, "        if self.cfg.stage == 3 and self.sample is None:\n            L[\"gathered\"] = gather_pack(self.plan, L[\"shards\"])\n        L[\"params\"] = shard_step(L[\"slices\"], self.cfg.gdt, self.hp, t, L[\"master\"], L[\"m\"], L[\"v\"],\n                                 self.cfg.pdt)\n        if self.cfg.stage == 3 and self.sample is None:\n            L[\"shards\"][self.cfg.owner] = L[\"params\"]\n", "        L[\"params\"] = shard_step(L[\"slices\"], self.cfg.gdt, self.hp, t, L[\"master\"], L[\"m\"], L[\"v\"],\n                                 self.cfg.pdt)\n        if self.cfg.stage == 3 and self.sample is None:\n            L[\"shards\"][self.cfg.owner] = L[\"params\"]\n            L[\"gathered\"] = gather_pack(self.plan, L[\"shards\"])\n"),
    ("stage3: owner shard not replaced", RUN, "            L[\"shards\"][self.cfg.owner] = L[\"params\"]\n", "            pass\n"),
    ("f64 adam: eps inside", C, "w[j] = w[j] - lr * mhat / (sqrt(vhat) + eps);", "w[j] = w[j] - lr * mhat / sqrt(vhat + eps);"),
]

def setup(workdir):
    global BASE
    BASE = os.path.join(os.path.abspath(workdir), 'repo_copy')
    if os.path.exists(BASE):
        shutil.rmtree(BASE)
    ign = shutil.ignore_patterns('.git', '_work', 'gpurun_out', '__pycache__', '.pytest_cache')
    shutil.copytree(R, BASE, ignore=ign)

def run(name, f, old, new):
    src = f'{BASE}/{f}'
    orig = open(src).read()
    if orig.count(old) != 1:
        return "NOT APPLIED"
    open(src, 'w').write(orig.replace(old, new))
    try:
        b = subprocess.run([sys.executable, '-c', 'from oracle import _build; _build.build()'], cwd=BASE,
                           capture_output=True, text=True)
        if b.returncode:
            return "BUILD FAILED"
        t = subprocess.run([sys.executable, '-m', 'pytest', 'tests/test_oracle_pins.py', '-x', '-q',
                            '-p', 'no:cacheprovider'], cwd=BASE, capture_output=True, text=True, timeout=900)
        if t.returncode == 0:
            return "SURVIVED"
        failed = [l for l in t.stdout.splitlines() if l.startswith('FAILED')]
        return "killed by " + (failed[0].split('::')[1].split(' ')[0] if failed else '?')
    finally:
        open(src, 'w').write(orig)

if __name__ == '__main__':
    if len(sys.argv) < 2:
        raise SystemExit(__doc__)
    setup(sys.argv[1])
    sel = sys.argv[2:]
    for name, f, old, new in MUTANTS:
        if sel and not any(s in name for s in sel):
            continue
        t0 = time.time()
        print(f"{name:34s} {run(name, f, old, new)}  ({time.time() - t0:.0f} s)", flush=True)
    # Equivalent by construction: "cast: fp16 max off" (65536 encodes as the
    # infinity pattern anyway), so it is expected to survive.
    subprocess.run([sys.executable, '-c', 'from oracle import _build; _build.build()'], cwd=BASE)
