"""The build's translation units and their flags (CPU only): every unit is
compiled for gfx950 with packed-fp32 instruction selection off; MFMA results
are kept in VGPRs in every unit but the head-dim-256 backward passes, whose
one-wave-per-SIMD kernels hold 256 accumulator registers in AGPRs."""

from attention_fa2_tiles_amd import build

VGPR_FORM = "-amdgpu-mfma-vgpr-form=1"


def test_common_flags():
    f = build.compile_flags()
    assert "--offload-arch=gfx950" in f
    i = f.index("-target-feature")
    assert f[i - 1:i + 3] == ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    assert VGPR_FORM not in " ".join(f)          # per unit, not global


def test_units_cover_every_part_once():
    us = build.units()
    names = [n for _, _, n in us]
    assert len(names) == len(set(names))
    for src, (macro, n) in build.PARTS.items():
        parts = [extra for s, extra, _ in us if s == src]
        assert len(parts) == n
        assert sorted(int(e[0].split("=")[1]) for e in parts) == list(range(n))
        assert all(e[0].startswith(f"-D{macro}=") for e in parts)
    for src in build.SOURCES:
        assert any(s == src for s, _, _ in us)


def test_vgpr_form_everywhere_but_the_agpr_parts():
    for src, extra, name in build.units():
        part = int(extra[0].split("=")[1]) if src in build.PARTS else None
        agpr = part is not None and part in build.AGPR_PARTS.get(src, ())
        assert (VGPR_FORM in " ".join(extra)) == (not agpr), name
    assert build.AGPR_PARTS == {"attn_bwd.hip": {5, 6, 7, 8}}
