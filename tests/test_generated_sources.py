"""The inline-assembly step sequences are generated: the committed include
must be exactly what gen_decode_asm.py writes (no hand edits, no stale
copy after a change to the generator)."""
import os
import shutil
import subprocess
import sys

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "head_latent_attention_11_amd", "csrc")


def test_asm_include_matches_its_generator(tmp_path):
    shutil.copy(os.path.join(CSRC, "gen_decode_asm.py"), tmp_path)
    subprocess.run([sys.executable, "gen_decode_asm.py"], cwd=tmp_path, check=True)
    with open(os.path.join(tmp_path, "decode_mfma_asm.inc"), "rb") as f:
        fresh = f.read()
    with open(os.path.join(CSRC, "decode_mfma_asm.inc"), "rb") as f:
        committed = f.read()
    assert fresh == committed
