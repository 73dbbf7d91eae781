"""The oracle's pins catch plausible mistakes.  Each case plants one mistake in a copy of the
oracle source (a dropped term, a wrong index or bound, a flipped comparison, a swapped operand),
builds it, and runs the pin suite against it in a child process: at least one pin must fail (a
crash of the mutant counts as caught).  The unmodified source, built the same way, passes.  Both
builds of the source are checked: the default float32 one and the float64 one.
CPU only; the mistakes live in temporary copies, never in the oracle itself."""

import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "nosa_oracle.c")

# name -> (original text, planted text); the original must occur exactly once.
MUTANTS = {
    "pool_divisor": ("Kp[((size_t)r * nsub + j) * d + c] = sum / (acc_t)sbs;",
                     "Kp[((size_t)r * nsub + j) * d + c] = sum / (acc_t)(sbs + 1);"),
    "pool_drops_last_token": ("for (int t = 0; t < sbs; t++)\n                    sum +=",
                              "for (int t = 0; t < sbs - 1; t++)\n                    sum +="),
    "scores_drop_a_head": ("for (int h = g * G; h < g * G + G; h++)",
                           "for (int h = g * G; h < g * G + G - (G > 1); h++)"),
    "scores_wrong_group": ("for (int h = g * G; h < g * G + G; h++)",
                           "for (int h = g; h < g + G; h++)"),
    "scores_min_pool": ("if (jj == 0 || u > best)", "if (jj == 0 || u < best)"),
    "topk_ties_to_higher_id": ("if (best < 0 || key[i] > key[best])", "if (best < 0 || key[i] >= key[best])"),
    "no_strict_eviction": ("candE[i] = prevE[i];", "candE[i] = 1;"),
    "window_off_by_one": ("const int fixed = (i < n_sink) || (i >= n_blocks - n_window);",
                          "const int fixed = (i < n_sink) || (i > n_blocks - n_window);"),
    "gamma_q_not_disjoint": ("candQ[i] = !inE[i];", "candQ[i] = 1;"),
    "cache_reversed_pairing": ("const int i = misses[m], blk = sel[i], slot = free_slots[m];",
                               "const int i = misses[m], blk = sel[i], slot = free_slots[nmiss - 1 - m];"),
    "cache_never_evicts": ("if (ob < 0 || !in_sel[ob])", "if (ob < 0)"),
    "attention_no_scale": ("z[i * bs + t] = sc * dot;", "z[i * bs + t] = dot;"),
    "attention_v_from_k": ("acc += z[i * bs + t] *\n                               elem(Vs,",
                           "acc += z[i * bs + t] *\n                               elem(Ks,"),
    "attention_not_normalised": ("out[(size_t)bh * d + c] = acc / l;\n            }\n        } else {",
                                 "out[(size_t)bh * d + c] = acc;\n            }\n        } else {"),
    "attention_wrong_kv_head": ("g = h / G;\n        const int64_t r = (int64_t)b * Hkv + g;\n        acc_t *z = malloc(sizeof(acc_t) * (size_t)T);",
                                "g = h % Hkv;\n        const int64_t r = (int64_t)b * Hkv + g;\n        acc_t *z = malloc(sizeof(acc_t) * (size_t)T);"),
    "masked_attention_ignores_mask": ("if (!mask[(size_t)r * n_blocks + t / bs]) {", "if (0) {"),
    "locality_divisor": ("gamma[r] = bad ? NAN : (double)both / (double)k;",
                         "gamma[r] = bad ? NAN : (double)both / (double)(k + 1);"),
}


def _build(text: str, tmp: str, name: str, f64: bool) -> str:
    src = os.path.join(tmp, name + ".c")
    lib = os.path.join(tmp, name + (".f64" if f64 else ".f32") + ".so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", *(["-DORACLE_F64"] if f64 else []),
                    src, "-o", lib, "-lm"], check=True)
    return lib


def _pins_pass(lib: str) -> bool:
    env = dict(os.environ, NOSA_ORACLE_LIBRARY=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x",
                        "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    return r.returncode == 0


@pytest.mark.parametrize("f64", [False, True], ids=["f32_build", "f64_build"])
def test_every_planted_mistake_fails_a_pin(f64):
    text = open(SRC).read()
    with tempfile.TemporaryDirectory() as tmp:
        libs = {"unmodified": _build(text, tmp, "unmodified", f64)}
        for name, (orig, planted) in MUTANTS.items():
            assert text.count(orig) == 1, "mutant %s: the original text must occur once" % name
            libs[name] = _build(text.replace(orig, planted), tmp, name, f64)
        with concurrent.futures.ThreadPoolExecutor(4) as ex:
            passed = dict(zip(libs, ex.map(_pins_pass, libs.values())))
    assert passed.pop("unmodified"), "the unmodified oracle must pass its pins"
    survivors = [n for n, ok in passed.items() if ok]
    assert not survivors, "planted mistakes no pin catches: %s" % survivors
